// Fused rotation + per-row INT4 quantization for row lengths n = m * p that are not
// powers of two: y = (H_m (x) H_p) x / sqrt(n), element a * p + b of a row being index
// (a, b) of the Kronecker product, H_p the Sylvester matrix in natural order and H_m a
// Paley matrix ("Rotations: QuaRot, SpinQuant and incoherence", section "Hadamard
// matrices": such lengths use the Kronecker product of a power-of-two Hadamard matrix with
// a small known one). The quantizer is the one of the power-of-two path: one absmax scale
// per row, max|y| / 7 floored at 1e-8, stored as fp32 or fp16, codes round half to even
// in [-8, 7], packed two per byte, low nibble first ("SpinQuant Guide: Learned Rotations
// for 4-Bit LLMs", step-size equation and the uniform_quantize_int4 listing).
//
// One workgroup of four waves per row (looping over rows when the grid is smaller):
//   0. once per workgroup: the operand-A table of H_m in LDS, 16-bit +-1 patterns in the
//      input's format, zero outside the m x m matrix, built from the quadratic character;
//   1. H_m runs on the matrix cores: for each block of 16 columns b, 16x16x32 MFMAs
//      multiply the m values X[.][b], gathered from HBM straight into operand registers
//      (fp32 inputs as three exact bf16 parts), with the table; the fp32 results go to
//      the LDS row buffer;
//   2. H_p: radix-2 butterflies over the bits of b, in passes through LDS (bits 4..8,
//      bits 9..10, then bits 0..3 on sixteen consecutive elements per thread, which also
//      takes the absmax);
//   3. the row absmax (wave shuffles, then LDS across the waves), the scale, and the
//      codes of each run of sixteen elements, written as 8-byte (packed) or 16-byte runs.
//
// Row buffer layout: element (a, b) at word a * rs + b + 4 (b / 16), i.e. four pad words
// after every sixteen elements, with rs = 4 (mod 16). The MFMA results (four rows 4 apart
// per lane group), the butterfly passes (lane groups on rows 4 apart, sixteen lanes on
// consecutive b) and the sixteen-element runs (20-word stride) then meet no LDS bank
// conflicts (runs of rows shorter than 256 elements meet at most 4-way ones).
//
// Everything is plain C++ against a context (lane, wave, barriers, LDS words, global
// loads and stores, shuffles, one MFMA), so the host emulator runs the same code.
#pragma once

#include "common.h"
#include "fwht_engine.h"

namespace rbq {

constexpr uint32_t kKronMaxWaves = 8;              // LDS slots for the per-wave maxima
constexpr uint32_t kKronMaxM = 256;                  // largest factor order the kernel takes
constexpr uint32_t kKronMaxKB = kKronMaxM / 32;      // 32-row K blocks of the MFMA
constexpr uint32_t kKronMaxN = 32768;
constexpr uint32_t kKronMinP = 16;
constexpr uint32_t kKronMaxP = 2048;

struct KronArgs {
  const void* x;
  int64_t row_stride;  // elements
  int64_t rows;
  void* codes;         // uint8 [rows, n/2] (packed) or int8 [rows, n]
  void* scales;        // [rows] fp32 or fp16
  float* rot32;        // optional [rows, n]
  uint32_t m, q, paley;  // paley 1: m = q + 1; paley 2: m = 2 (q + 1); 3: Goethals-Seidel, m = 4 q
  uint32_t p_log;
  uint32_t opts;         // OPT_PACKED, OPT_SCALE_F16
  uint32_t qr[8];        // Paley: bit d is set iff d is a nonzero square modulo q (q < 256);
                         // Goethals-Seidel: the first rows of A, B, C, D, two words each
  float sqrtn;           // sqrt(n) rounded to float
  float inv_sqrtn;       // 1 / sqrt(n) rounded to float
  uint32_t rs;           // LDS words per row a of the [m][p] buffer (p + 4)
  uint32_t hs;           // LDS words per row of the operand table (16 KB + 4)
  uint32_t tab0;         // LDS word offset of the table
  uint32_t red0;         // LDS word offset of the per-wave maxima (up to 8 waves)
};

// LDS words a launch needs (the row buffer, the table, the cross-wave maxima)
RBQ_HD uint32_t kron_lds_words(uint32_t m, uint32_t p_log, uint32_t* rs, uint32_t* hs,
                               uint32_t* tab0, uint32_t* red0) {
  const uint32_t p = 1u << p_log;
  const uint32_t mb = (m + 15) / 16, kb = (m + 31) / 32;
  const uint32_t padded = p + p / 4;
  *rs = padded + ((4u + 16u - (padded & 15u)) & 15u);  // = 4 (mod 16)
  *hs = kb * 16 + 4;
  *tab0 = m * *rs;
  *red0 = *tab0 + mb * 16 * *hs;
  return *red0 + kKronMaxWaves;
}

// Waves per workgroup and operand blocks per gather chunk for KB K blocks of the MFMA.
// Rows with m <= 32 in a 16-bit format take 8 waves with chunks of 4 blocks: their
// registers then fit 4 waves per SIMD, so two workgroups of 8 waves share a CU and twice
// as many gathers are in flight. Orders 161 to 192 (six K blocks) in a 16-bit format also
// take 8 waves (one block per chunk): their LDS (operand table and row buffer) leaves room
// for one workgroup per CU, and 8 waves give each SIMD two within 256 VGPRs. Otherwise 4
// waves with chunks of 8 / KB blocks.
template <int IN, int KB>
constexpr uint32_t kron_waves() { return (IN != IN_F32 && (KB == 1 || KB == 6)) ? 8u : 4u; }

template <int IN, int KB>
constexpr int kron_chunk() {
  if (IN == IN_F32 || KB > 8) return 1;
  return KB == 1 ? (kron_waves<IN, KB>() == 8u ? 4 : 8) : 8 / KB;
}

// quadratic character of GF(q) from the square mask: 0, +1 (nonzero square) or -1
RBQ_HD int kron_chi(const uint32_t* qr, uint32_t d) {
  if (d == 0) return 0;
  return ((qr[d >> 5] >> (d & 31)) & 1u) ? 1 : -1;
}

// Entry (i, j) of block (R, C) of the Goethals-Seidel array
//   [[ A, BR, CR, DR], [-BR, A, D^T R, -C^T R], [-CR, -D^T R, A, B^T R], [-DR, C^T R, -B^T R, A]]
// on circulants of order q with first rows in qr (two words per matrix). With
// X[i][j] = x[(j - i) mod q]: X = x[(j - i)], X R = x[(q - 1 - i - j)], X^T R = x[(i + j + 1)].
RBQ_HD int gs_entry(uint32_t q, const uint32_t* qr, uint32_t r, uint32_t c) {
  // per block b = 4 R + C, two bits each: the matrix (0..3 = A..D) and the form
  // (0: X, 1: X R, 2: X^T R); one bit each: a negative sign. Rows of the array:
  //   mat  0 1 2 3 | 1 0 3 2 | 2 3 0 1 | 3 2 1 0
  //   form 0 1 1 1 | 1 0 2 2 | 1 2 0 2 | 1 2 2 0
  //   neg  0 0 0 0 | 1 0 0 1 | 1 1 0 0 | 1 0 1 0
  constexpr uint32_t kMat = 0x1b4eb1e4u, kForm = 0x2989a154u, kNeg = 0x5390u;
  const uint32_t R = r / q, C = c / q, i = r - R * q, j = c - C * q;
  const uint32_t b = 4 * R + C;
  const uint32_t mat = (kMat >> (2 * b)) & 3u, form = (kForm >> (2 * b)) & 3u;
  uint32_t t;
  if (form == 0) t = (j + q - i) % q;
  else if (form == 1) t = (2 * q - 1 - i - j) % q;
  else t = (i + j + 1) % q;
  const uint32_t w = qr[2 * mat + (t >> 5)];
  const int v = ((w >> (t & 31)) & 1u) ? 1 : -1;
  return ((kNeg >> b) & 1u) ? -v : v;
}

// Entry (r, c) of the small factor. Paley I: I + [[0, 1...], [-1..., Q]] with
// Q[a][b] = chi(a - b). Paley II: the conference matrix [[0, 1...], [1..., Q]] with each
// 0 replaced by [[1, -1], [-1, -1]] and each +-1 by +-[[1, 1], [1, -1]]. Kind 3: the
// Goethals-Seidel array above.
RBQ_HD int paley_entry(uint32_t paley, uint32_t q, const uint32_t* qr, uint32_t r, uint32_t c) {
  if (paley == 3) return gs_entry(q, qr, r, c);
  if (paley == 1) {
    if (r == c || r == 0) return 1;
    if (c == 0) return -1;
    return kron_chi(qr, (r + q - c) % q);
  }
  const uint32_t R = r >> 1, C = c >> 1;
  if (R == C) return ((r | c) & 1u) ? -1 : 1;
  const int v = (R == 0 || C == 0) ? 1 : kron_chi(qr, (R + q - C) % q);
  return (r & c & 1u) ? -v : v;
}

// In-register Sylvester transform of G bits over v[0 .. 2^G) (natural order)
template <int G>
RBQ_HD void kron_fwht_regs(float* v) {
  static_for<0, G>([&](auto T) {
    constexpr int h = 1 << T.value;
    static_for<0, (1 << G) / 2>([&](auto I) {
      constexpr int lo = ((I.value >> T.value) << (T.value + 1)) | (I.value & (h - 1));
      const float a = v[lo], b = v[lo + h];
      v[lo] = a + b;
      v[lo + h] = a - b;
    });
  });
}

// One LDS pass of H_p over the G bits [O, O + G) of b for every row a (compile-time bit
// positions, so the element offsets are immediates of the LDS instructions). A job is one
// wave: lanes 0..15 take sixteen consecutive b (bits 0..3), lane groups 1..3 the rows 4,
// 8 and 12 below; the job index runs over the groups of sixteen rows, the first row of
// the group, the bits of b above the pass and those between bit 4 and bit O.
template <int O, int G, uint32_t W, class Ctx>
RBQ_HD void kron_pass(Ctx& c, uint32_t m, uint32_t P, uint32_t rs) {
  const uint32_t hib = P - O - G;
  const uint32_t nlh = 1u << (O - 4);
  const uint32_t nhi = 1u << hib;
  const uint32_t njobs = ((m + 15) / 16) * 4 * nhi * nlh;
  const uint32_t lowlo = c.lane & 15u, t = c.lane >> 4;
  for (uint32_t j = c.wave; j < njobs; j += W) {
    const uint32_t lh = j & (nlh - 1u);
    const uint32_t r = j >> (O - 4);
    const uint32_t hi = r & (nhi - 1u);
    const uint32_t r2 = r >> hib;
    const uint32_t a = 16 * (r2 >> 2) + (r2 & 3u) + 4 * t;
    if (a < m) {
      const uint32_t b0 = lowlo | (lh << 4) | (hi << (O + G));
      const uint32_t base = a * rs + b0 + ((b0 >> 4) << 2);
      // element b0 + (i << O) sits (i << O) + (i << (O - 2)) words after b0's
      float v[1 << G];
      static_for<0, (1 << G)>([&](auto I) {
        v[I.value] = c.lds_load(base + ((uint32_t)I.value << O) + ((uint32_t)I.value << (O - 2)));
      });
      kron_fwht_regs<G>(v);
      static_for<0, (1 << G)>([&](auto I) {
        c.lds_store(base + ((uint32_t)I.value << O) + ((uint32_t)I.value << (O - 2)), v[I.value]);
      });
    }
  }
}

// H_m on the matrix cores: Y[a][b] = sum_a' H_m[a][a'] X[a'][b] as D = A B, with A = H_m
// (rows a, K = a') from the LDS table and B = X (K = a', columns b) gathered from HBM
// straight into operand registers; rows a' >= m read row m - 1, which the zero columns of
// the table cancel. Each wave takes the blocks of 16 columns nb = wave, wave + W, ... (W waves) in
// chunks of NBC blocks: the operands of a chunk are gathered before its MFMAs, so one
// memory latency covers the chunk, and the first chunk of the next row is gathered while
// the current row is transformed and quantized. The fp32 results go to the row buffer.
template <int IN, int KB>
struct KronFrag {
  static constexpr int NBC = kron_chunk<IN, KB>();  // blocks per chunk
  // the raw gathered values (one 16-bit or fp32 element per register): they are packed
  // or split into MFMA operands only where used, so the loads of a prefetch stay in
  // flight until then
  uint32_t r[NBC][KB][8];
};

// byte offsets, from the row's start, of the eight K rows a lane gathers for K block kb
// and column col (rows clamped to m - 1)
template <int IN, int KB>
struct KronGatherOffsets {
  uint32_t off[KB][8];
};

template <int IN, int KB, class Ctx>
RBQ_HD KronGatherOffsets<IN, KB> kron_gather_offsets(Ctx& c, const KronArgs& a) {
  constexpr uint32_t ESZ = (IN == IN_F32) ? 4 : 2;
  const uint32_t m = a.m, p = 1u << a.p_log;
  const uint32_t col = c.lane & 15u, grp = c.lane >> 4;
  KronGatherOffsets<IN, KB> g;
  static_for<0, KB>([&](auto KBI) {
    static_for<0, 8>([&](auto I) {
      uint32_t ap = 32 * KBI.value + 8 * grp + I.value;
      ap = ap < m ? ap : m - 1;
      g.off[KBI.value][I.value] = (ap * p + col) * ESZ;  // n * ESZ < 2^17
    });
  });
  return g;
}

template <int IN, int KB, class Ctx>
RBQ_HD void kron_gather(Ctx& c, const KronArgs& a, const KronGatherOffsets<IN, KB>& g, const char* xr,
                        uint32_t nb0, KronFrag<IN, KB>& f) {
  using F = KronFrag<IN, KB>;
  constexpr uint32_t ESZ = (IN == IN_F32) ? 4 : 2;
  const uint32_t NB = (1u << a.p_log) >> 4;
  static_for<0, F::NBC>([&](auto JJ) {
    const uint32_t nb = nb0 + kron_waves<IN, KB>() * JJ.value;
    if (nb < NB) {
      const char* xb = xr + nb * 16 * ESZ;  // uniform: the block's first column
      static_for<0, KB>([&](auto KBI) {
        static_for<0, 8>([&](auto I) {
          // a 32-bit offset from a uniform base (kept opaque so that it is not widened
          // to 64 bits ahead of time)
          const uint32_t o = c.opaque(g.off[KBI.value][I.value]);
          if constexpr (IN == IN_F32) f.r[JJ.value][KBI.value][I.value] = c.template load<uint32_t>(xb + o);
          else f.r[JJ.value][KBI.value][I.value] = c.template load<uint16_t>(xb + o);
        });
      });
    }
  });
}

template <int IN, int KB, class Ctx>
RBQ_HD void kron_mma_store(Ctx& c, const KronArgs& a, uint32_t nb0, const KronFrag<IN, KB>& f, uint32_t mb_lo,
                           uint32_t mb_hi) {
  using F = KronFrag<IN, KB>;
  constexpr int NPART = (IN == IN_F32) ? 3 : 1;  // bf16 parts of an MFMA operand
  const uint32_t NB = (1u << a.p_log) >> 4;
  const uint32_t col = c.lane & 15u, grp = c.lane >> 4;
  static_for<0, F::NBC>([&](auto JJ) {
    const uint32_t nb = nb0 + kron_waves<IN, KB>() * JJ.value;
    if (nb < NB) {
      // operand B of each K block: element i of the lane's eight in half i % 2 of word i / 2
      uint32_t bf[KB][NPART][4];
      static_for<0, KB>([&](auto KBI) {
        static_for<0, 4>([&](auto W) {
          uint32_t h[2][NPART];
          static_for<0, 2>([&](auto H) {
            const uint32_t u = f.r[JJ.value][KBI.value][2 * W.value + H.value];
            if constexpr (IN == IN_F32) {
              // x = hi + mid + lo exactly, each a bfloat16 (truncations of x and of the
              // remainders: 8 + 8 + 8 significant bits)
              const float x = bits_f32(u);
              const float xh = bits_f32(u & 0xFFFF0000u);
              const float r1 = x - xh;
              const float xm = bits_f32(f32_bits(r1) & 0xFFFF0000u);
              const float r2 = r1 - xm;
              h[H.value][0] = u >> 16;
              h[H.value][1] = f32_bits(xm) >> 16;
              h[H.value][2] = f32_bits(r2) >> 16;
            } else {
              h[H.value][0] = u;
            }
          });
          static_for<0, NPART>([&](auto Q) { bf[KBI.value][Q.value][W.value] = h[0][Q.value] | (h[1][Q.value] << 16); });
        });
      });
      const uint32_t bcol = nb * 16 + col;
      const uint32_t cw = bcol + ((bcol >> 4) << 2);  // word of column bcol within a row
      for (uint32_t mb = mb_lo; mb < mb_hi; ++mb) {
        float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        const uint32_t trow = a.tab0 + (16 * mb + col) * a.hs + 4 * grp;
        static_for<0, KB>([&](auto KBI) {
          constexpr int kb = KBI.value;
          const f32x4 t4 = c.lds_load4(trow + 16 * kb);
          const uint32_t af[4] = {f32_bits(t4.x), f32_bits(t4.y), f32_bits(t4.z), f32_bits(t4.w)};
          // smallest parts first
          static_for<0, NPART>([&](auto Q) { c.template mfma16x16x32<IN>(af, bf[kb][NPART - 1 - Q.value], acc); });
        });
        static_for<0, 4>([&](auto J) {
          const uint32_t ar = 16 * mb + 4 * grp + J.value;
          if (ar < a.m) c.lds_store(ar * a.rs + cw, acc[J.value]);
        });
      }
    }
  });
}

// sixteen consecutive words at a 16-byte aligned word index (four 128-bit LDS reads)
template <class Ctx>
RBQ_HD void kron_load16(Ctx& c, uint32_t base, float (&v)[16]) {
  static_for<0, 4>([&](auto Q) {
    const f32x4 t = c.lds_load4(base + 4 * Q.value);
    v[4 * Q.value] = t.x;
    v[4 * Q.value + 1] = t.y;
    v[4 * Q.value + 2] = t.z;
    v[4 * Q.value + 3] = t.w;
  });
}

// The rows of one workgroup, for K blocks KB = ceil(m / 32) of the MFMA
template <int IN, int KB, class Ctx>
RBQ_HD void kron_rows(Ctx& c, const KronArgs& a, uint32_t wg, uint32_t grid) {
  constexpr uint32_t ESZ = (IN == IN_F32) ? 4 : 2;
  constexpr uint32_t W = kron_waves<IN, KB>(), NT = 64 * W;
  using F = KronFrag<IN, KB>;
  const uint32_t tid = c.wave * 64u + c.lane;
  const uint32_t m = a.m, P = a.p_log, p = 1u << P, n = m << P;
  const uint32_t NB = p >> 4;
  const uint32_t rs = a.rs;
  const bool packed = (a.opts & OPT_PACKED) != 0;
  const bool scale_f16 = (a.opts & OPT_SCALE_F16) != 0;
  const uint32_t nrun = n >> 4;

  const KronGatherOffsets<IN, KB> go = kron_gather_offsets<IN, KB>(c, a);
  auto row_ptr = [&](int64_t r) { return (const char*)a.x + r * a.row_stride * (int64_t)ESZ; };
  F pre;  // the first chunk of this wave's columns for the next row
  // With fewer column blocks than waves (NB < W), R = W / NB waves share each block, each
  // taking a range of the 16-row blocks mb of H_m; waves whose range is empty take no block.
  const uint32_t MB = (m + 15) / 16;
  const uint32_t R = NB < W ? W / NB : 1u;
  const uint32_t part = c.wave / (W / R);
  const uint32_t mb_lo = part * MB / R, mb_hi = (part + 1) * MB / R;
  const uint32_t nb_first = mb_lo < mb_hi ? c.wave % (W / R) : NB;
  if ((int64_t)wg < a.rows) kron_gather<IN, KB>(c, a, go, row_ptr(wg), nb_first, pre);

  for (int64_t row = wg; row < a.rows; row += grid) {
    const char* xr = row_ptr(row);

    // ---- 1. H_m on the matrix cores
    kron_mma_store<IN, KB>(c, a, nb_first, pre, mb_lo, mb_hi);
    for (uint32_t nb0 = nb_first + W * F::NBC; nb0 < NB; nb0 += W * F::NBC) {
      F f;
      kron_gather<IN, KB>(c, a, go, xr, nb0, f);
      kron_mma_store<IN, KB>(c, a, nb0, f, mb_lo, mb_hi);
    }
    if (row + grid < a.rows) kron_gather<IN, KB>(c, a, go, row_ptr(row + grid), nb_first, pre);
    c.barrier_lds();

    // ---- 2. H_p over the bits of b above bit 3: bits 4..8, then bits 9..10
    switch (P) {
      case 5: kron_pass<4, 1, W>(c, m, P, rs); break;
      case 6: kron_pass<4, 2, W>(c, m, P, rs); break;
      case 7: kron_pass<4, 3, W>(c, m, P, rs); break;
      case 8: kron_pass<4, 4, W>(c, m, P, rs); break;
      case 9: case 10: case 11: kron_pass<4, 5, W>(c, m, P, rs); break;
      default: break;
    }
    if (P > 4) c.barrier_lds();
    if (P == 10) kron_pass<9, 1, W>(c, m, P, rs);
    if (P == 11) kron_pass<9, 2, W>(c, m, P, rs);
    if (P > 9) c.barrier_lds();

    // ---- 2b. bits 0..3 on sixteen consecutive elements per run, and the row's absmax
    float mx = 0.0f;
    for (uint32_t s = tid; s < nrun; s += NT) {
      const uint32_t base = (s >> (P - 4)) * rs + (s & ((p >> 4) - 1u)) * 20u;
      float v[16];
      kron_load16(c, base, v);
      kron_fwht_regs<4>(v);
      static_for<0, 16>([&](auto I) { mx = fmaxf(mx, fabsf(v[I.value])); });
      static_for<0, 4>([&](auto Q) {
        constexpr int q4 = 4 * Q.value;
        c.lds_store4(base + q4, f32x4{v[q4], v[q4 + 1], v[q4 + 2], v[q4 + 3]});
      });
    }
    static_for<0, 6>([&](auto B) { mx = fmaxf(mx, c.shfl_xor(mx, 1 << B.value)); });
    if (c.lane == 0) c.lds_store(a.red0 + c.wave, mx);
    c.barrier_lds();

    // ---- 3. scale and codes, one run of sixteen consecutive elements at a time
    float mu = 0.0f;
    static_for<0, (int)W>([&](auto WV) { mu = fmaxf(mu, c.lds_load(a.red0 + WV.value)); });
    const float qmax = 7.0f;
    float sc = mu / (qmax * a.sqrtn);
    sc = fmaxf(sc, 1e-8f);
    float s_st = sc;
    uint32_t h16 = 0;
    if (scale_f16) { h16 = f32_to_f16(sc); s_st = f16_to_f32(h16); }
    const float mk = (s_st == 0.0f) ? 0.0f : 1.0f / (s_st * a.sqrtn);
    if (tid == 0) {
      if (scale_f16) c.template store<uint16_t>((uint16_t*)a.scales + row, (uint16_t)h16);
      else c.template store<float>((float*)a.scales + row, s_st);
    }
    // |u * mk| <= mu * mk; unless a subnormal fp16 scale sits far below max / 7, codes
    // cannot leave [-7, 7] and the clamp is skipped
    const bool clamp = mu * mk > qmax + 0.25f;
    auto code_runs = [&](auto CL) {
      constexpr bool CLAMP = decltype(CL)::value != 0;
      for (uint32_t s = tid; s < nrun; s += NT) {
        const uint32_t base = (s >> (P - 4)) * rs + (s & ((p >> 4) - 1u)) * 20u;
        const uint32_t el = s << 4;  // the run's first element: a * p + b0
        float v[16];
        kron_load16(c, base, v);
        auto code = [&](float u) {
          float qv = fmaf(u, mk, kMagic);
          if constexpr (CLAMP) qv = fminf(fmaxf(qv, kMagic - qmax - 1.0f), kMagic + qmax);
          return f32_bits(qv);
        };
        if (packed) {
          uint32_t w[2] = {0u, 0u};
          static_for<0, 16>([&](auto I) { w[I.value / 8] = alignbit(code(v[I.value]), w[I.value / 8], 4); });
          c.template store<u32x2>((uint8_t*)a.codes + row * (int64_t)(n / 2) + el / 2, u32x2{w[0], w[1]});
        } else {
          uint32_t w[4] = {0u, 0u, 0u, 0u};
          static_for<0, 16>([&](auto I) { w[I.value / 4] = alignbit(code(v[I.value]), w[I.value / 4], 8); });
          c.template store<u32x4>((uint8_t*)a.codes + row * (int64_t)n + el, u32x4{w[0], w[1], w[2], w[3]});
        }
        if (a.rot32) {
          float* dst = a.rot32 + row * (int64_t)n + el;
          static_for<0, 4>([&](auto Q) {
            constexpr int q4 = 4 * Q.value;
            c.template store<u32x4>(dst + q4, u32x4{f32_bits(v[q4] * a.inv_sqrtn), f32_bits(v[q4 + 1] * a.inv_sqrtn),
                                                    f32_bits(v[q4 + 2] * a.inv_sqrtn), f32_bits(v[q4 + 3] * a.inv_sqrtn)});
          });
        }
      }
    };
    if (clamp) code_runs(IC<1>{}); else code_runs(IC<0>{});
    // the next row's MFMA results overwrite the buffer the runs above read
    c.barrier_lds();
  }
}

// KS 1: the kernel for one K block (m <= 32); KS 0: two to five (m <= 160); KS 2: six
// (m <= 192); KS 3: seven and eight (m <= 256). Each range is its own kernel, so the
// register budget and wave count of one does not weigh on the others.
template <int IN, int KS>
constexpr uint32_t kron_body_waves() {
  return KS == 1 ? kron_waves<IN, 1>() : KS == 2 ? kron_waves<IN, 6>() : KS == 3 ? kron_waves<IN, 7>()
                                                                                  : kron_waves<IN, 2>();
}

template <int IN, int KS, class Ctx>
RBQ_HD void kron_quant_body(Ctx& c, const KronArgs& a, uint32_t wg, uint32_t grid) {
  constexpr uint32_t NT = 64 * kron_body_waves<IN, KS>();
  const uint32_t tid = c.wave * 64u + c.lane;
  const uint32_t m = a.m;
  const uint32_t MB = (m + 15) / 16, KB = (m + 31) / 32;
  const uint32_t hs = a.hs, tab0 = a.tab0;

  // ---- 0. operand table: row r, words w hold H_m[r][2w] (low half) and H_m[r][2w + 1]
  {
    const uint32_t one = (IN == IN_F16) ? 0x3C00u : 0x3F80u;
    const uint32_t wpr = KB * 16;
    for (uint32_t w = tid; w < MB * 16 * wpr; w += NT) {
      const uint32_t r = w / wpr, cw = w - r * wpr;
      uint32_t bits = 0;
      for (uint32_t h = 0; h < 2; ++h) {
        const uint32_t cc = 2 * cw + h;
        if (r < m && cc < m) {
          const int e = paley_entry(a.paley, a.q, a.qr, r, cc);
          bits |= (e > 0 ? one : (one | 0x8000u)) << (16 * h);
        }
      }
      c.lds_store(tab0 + r * hs + cw, bits_f32(bits));
    }
  }
  c.barrier();  // the table is read by every wave's MFMAs

  if constexpr (KS == 1) {
    kron_rows<IN, 1>(c, a, wg, grid);
  } else if constexpr (KS == 0) {
    switch (KB) {
      case 2: kron_rows<IN, 2>(c, a, wg, grid); break;
      case 3: kron_rows<IN, 3>(c, a, wg, grid); break;
      case 4: kron_rows<IN, 4>(c, a, wg, grid); break;
      default: kron_rows<IN, 5>(c, a, wg, grid); break;
    }
  } else if constexpr (KS == 2) {
    kron_rows<IN, 6>(c, a, wg, grid);
  } else {
    if (KB == 7) kron_rows<IN, 7>(c, a, wg, grid);
    else kron_rows<IN, 8>(c, a, wg, grid);
  }
}

}  // namespace rbq
