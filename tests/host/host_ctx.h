// Host execution context for the kernel bodies: one std::thread per GPU lane, with LDS,
// workgroup barriers, wave-level synchronisation, lane shuffles and the MFMAs emulated,
// and every global and LDS access bounds-checked against registered buffers.
#pragma once

#include <barrier>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <memory>
#include <vector>

#include "../../rotation_bit_quantization_fwht_amd/csrc/fwht_engine.h"

namespace rbq {

struct Buf { const char* lo; const char* hi; const char* name; };
static std::vector<Buf> g_bufs;

static void check_ptr(const void* p, size_t n, const char* what) {
  const char* c = (const char*)p;
  for (auto& b : g_bufs)
    if (c >= b.lo && c + n <= b.hi) return;
  fprintf(stderr, "OUT OF BOUNDS %s access at %p (+%zu)\n", what, p, n);
  std::abort();
}

struct WgShared {
  std::vector<float> lds;
  std::barrier<> wg;
  std::vector<std::unique_ptr<std::barrier<>>> wave_bar;
  std::vector<std::vector<float>> shfl;
  std::vector<std::vector<float>> mfma_b;  // per wave: 64 lanes x 8 operand-B values
  std::vector<std::vector<float>> mfma_a;  // per wave: 64 lanes x 8 operand-A values
  WgShared(size_t lds_words, int nthreads, int nwaves)
      : lds(lds_words, -12345.0f), wg(nthreads) {
    for (int w = 0; w < nwaves; ++w) {
      wave_bar.emplace_back(new std::barrier<>(64));
      shfl.emplace_back(64, 0.0f);
      mfma_b.emplace_back(64 * 8, 0.0f);
      mfma_a.emplace_back(64 * 8, 0.0f);
    }
  }
};

static constexpr HadamardA kHA = make_hadamard_a();

static float half16(uint32_t h, int in) { return in == IN_F16 ? f16_to_f32(h) : bf16_to_f32(h); }

struct HostCtx {
  uint32_t lane, wave;
  WgShared* s;
  void refresh_ids() {}
  void barrier() { s->wg.arrive_and_wait(); }
  void barrier_lds() { s->wg.arrive_and_wait(); }
  uint32_t opaque(uint32_t v) { return v; }
  void wave_sync() { s->wave_bar[wave]->arrive_and_wait(); }
  float shfl_xor(float v, int m) {
    s->shfl[wave][lane] = v;
    s->wave_bar[wave]->arrive_and_wait();
    float r = s->shfl[wave][lane ^ (uint32_t)m];
    s->wave_bar[wave]->arrive_and_wait();
    return r;
  }
  template <int M> float shfl_xor_c(float v) { return shfl_xor(v, M); }
  template <class T> T load(const void* p) {
    check_ptr(p, sizeof(T), "load");
    if ((uintptr_t)p % alignof(T)) { fprintf(stderr, "MISALIGNED load\n"); std::abort(); }
    T v; memcpy(&v, p, sizeof(T)); return v;
  }
  template <class T> void store(void* p, T v) {
    check_ptr(p, sizeof(T), "store");
    if ((uintptr_t)p % alignof(T)) { fprintf(stderr, "MISALIGNED store\n"); std::abort(); }
    memcpy(p, &v, sizeof(T));
  }
  void lds_store(uint32_t i, float v) {
    if (i >= s->lds.size()) { fprintf(stderr, "LDS OOB store %u/%zu\n", i, s->lds.size()); std::abort(); }
    s->lds[i] = v;
  }
  float lds_load(uint32_t i) {
    if (i >= s->lds.size()) { fprintf(stderr, "LDS OOB load %u/%zu\n", i, s->lds.size()); std::abort(); }
    return s->lds[i];
  }
  f32x4 lds_load4(uint32_t i) {
    if (i % 4) { fprintf(stderr, "MISALIGNED LDS load4 %u\n", i); std::abort(); }
    return f32x4{lds_load(i), lds_load(i + 1), lds_load(i + 2), lds_load(i + 3)};
  }
  void lds_store4(uint32_t i, f32x4 v) {
    if (i % 4) { fprintf(stderr, "MISALIGNED LDS store4 %u\n", i); std::abort(); }
    lds_store(i, v.x); lds_store(i + 1, v.y); lds_store(i + 2, v.z); lds_store(i + 3, v.w);
  }
  template <int IN> void widen(uint32_t w, float& a, float& b) {
    if (IN == IN_BF16) { a = bf16_to_f32(w & 0xFFFFu); b = bf16_to_f32(w >> 16); }
    else { a = f16_to_f32(w & 0xFFFFu); b = f16_to_f32(w >> 16); }
  }
  // emulation of the 16x16x32 MFMA with the constant operand A of plan.h:
  // D[i][j] = sum_k A_m[i][k] B[k][j]; A: lane l = row l%16, k = 8 (l/16) + v;
  // B: lane l = column l%16, k = 8 (l/16) + v; D: lane l, reg r = D[4 (l/16) + r][l%16]
  template <int IN> void hadamard32(const uint32_t (&b)[4], int m, float (&d)[4]) {
    std::vector<float>& buf = s->mfma_b[wave];
    for (int v = 0; v < 8; ++v) buf[lane * 8 + v] = half16((b[v / 2] >> (16 * (v % 2))) & 0xFFFFu, IN);
    s->wave_bar[wave]->arrive_and_wait();
    const int fmt = (IN == IN_F16) ? 1 : 0;
    const int j = (int)lane % 16;
    for (int r = 0; r < 4; ++r) {
      const int i = 4 * ((int)lane / 16) + r;
      float acc = 0.0f;
      for (int g = 0; g < 4; ++g)
        for (int v = 0; v < 8; ++v) {
          const uint32_t aw = kHA.w[fmt][m][i + 16 * g][v / 2];
          const float av = half16((aw >> (16 * (v % 2))) & 0xFFFFu, IN);
          acc += av * buf[(j + 16 * g) * 8 + v];
        }
      d[r] = acc;
    }
    s->wave_bar[wave]->arrive_and_wait();
  }
  // emulation of one 16x16x32 MFMA with both operands from the lanes' registers:
  // D[i][j] += sum_k A[i][k] B[k][j], layouts as in hadamard32; bf16 unless IN is IN_F16
  template <int IN> void mfma16x16x32(const uint32_t (&a)[4], const uint32_t (&b)[4], float (&d)[4]) {
    const int fmt = (IN == IN_F16) ? IN_F16 : IN_BF16;
    std::vector<float>& ab = s->mfma_a[wave];
    std::vector<float>& bb = s->mfma_b[wave];
    for (int v = 0; v < 8; ++v) {
      ab[lane * 8 + v] = half16((a[v / 2] >> (16 * (v % 2))) & 0xFFFFu, fmt);
      bb[lane * 8 + v] = half16((b[v / 2] >> (16 * (v % 2))) & 0xFFFFu, fmt);
    }
    s->wave_bar[wave]->arrive_and_wait();
    const int j = (int)lane % 16;
    for (int r = 0; r < 4; ++r) {
      const int i = 4 * ((int)lane / 16) + r;
      float acc = d[r];
      for (int g = 0; g < 4; ++g)
        for (int v = 0; v < 8; ++v) acc += ab[(i + 16 * g) * 8 + v] * bb[(j + 16 * g) * 8 + v];
      d[r] = acc;
    }
    s->wave_bar[wave]->arrive_and_wait();
  }
  template <int IN> void widen_butterfly(uint32_t w, float& a, float& b) {
    float x0, x1;
    widen<IN>(w, x0, x1);
    a = x0 + x1;
    b = x0 - x1;
  }
};

}  // namespace rbq
