// Host execution of the rotation + INT4 quantizer for row lengths that are not powers of
// two (the workgroup body of kron_engine.h, the same template code the HIP kernel runs),
// with the kernel arguments filled by the library's own host logic (kron_factor.h). Every
// global and LDS access is bounds-checked (host_ctx.h). Used by tests/test_host_emulator.py.
//
// usage: kron_emu IN n rows opts x.bin row_stride codes.bin scales.bin [rot.bin]
// opts: 1 packed codes, 2 fp16 scales. Prints "m p paley q lds_words" on success.
#include <cstdio>
#include <cstdlib>
#include <string>
#include <thread>
#include <vector>

#include "../../rotation_bit_quantization_fwht_amd/csrc/kron_engine.h"
#include "../../rotation_bit_quantization_fwht_amd/csrc/kron_factor.h"
#include "host_ctx.h"

using namespace rbq;

// the kernel the library launches: one K block (m <= 32) or more, each with its waves
template <int IN, int KS>
static void run_ks(const KronArgs& a, uint32_t words, uint32_t grid) {
  constexpr uint32_t W = kron_body_waves<IN, KS>();
  for (uint32_t wg = 0; wg < grid; ++wg) {
    WgShared sh(words, (int)(64 * W), (int)W);
    std::vector<std::thread> th;
    for (uint32_t t = 0; t < 64 * W; ++t)
      th.emplace_back([&, t] {
        HostCtx c{t & 63u, t >> 6, &sh};
        kron_quant_body<IN, KS>(c, a, wg, grid);
      });
    for (auto& x : th) x.join();
  }
}

template <int IN>
static void run(const KronArgs& a, uint32_t words, uint32_t grid) {
  if (a.m <= 32u) run_ks<IN, 1>(a, words, grid);
  else if (a.m <= 160u) run_ks<IN, 0>(a, words, grid);
  else if (a.m <= 192u) run_ks<IN, 2>(a, words, grid);
  else run_ks<IN, 3>(a, words, grid);
}

static std::vector<char> read_file(const char* path) {
  FILE* f = fopen(path, "rb");
  if (!f) { perror(path); std::exit(2); }
  fseek(f, 0, SEEK_END); long n = ftell(f); fseek(f, 0, SEEK_SET);
  std::vector<char> v(n);
  if (n && fread(v.data(), 1, n, f) != (size_t)n) { perror("read"); std::exit(2); }
  fclose(f);
  return v;
}

static void write_file(const char* path, const void* p, size_t n) {
  FILE* f = fopen(path, "wb");
  if (!f) { perror(path); std::exit(2); }
  if (n) fwrite(p, 1, n, f);
  fclose(f);
}

int main(int argc, char** argv) {
  if (argc < 9) { fprintf(stderr, "bad args\n"); return 2; }
  const int in = atoi(argv[1]);
  const long long n = atoll(argv[2]), rows = atoll(argv[3]);
  const unsigned opts = (unsigned)atoi(argv[4]);
  std::vector<char> x = read_file(argv[5]);
  const long long row_stride = atoll(argv[6]);
  KronArgs a{};
  const uint32_t words = kron_setup(n, a);
  if (words == 0) { fprintf(stderr, "unsupported n\n"); return 3; }
  auto alloc = [](size_t bytes) { return (char*)aligned_alloc(64, ((bytes + 63) / 64) * 64 + 64); };
  char* xb = alloc(x.size());
  memcpy(xb, x.data(), x.size());
  const size_t code_bytes = (size_t)rows * ((opts & OPT_PACKED) ? n / 2 : n);
  const size_t scale_bytes = (size_t)rows * ((opts & OPT_SCALE_F16) ? 2 : 4);
  const size_t rot_bytes = (size_t)rows * n * 4;
  char* codes = alloc(code_bytes);
  char* scales = alloc(scale_bytes);
  char* rotb = alloc(rot_bytes);
  memset(codes, 0xEE, code_bytes); memset(scales, 0xEE, scale_bytes); memset(rotb, 0xEE, rot_bytes);
  g_bufs.push_back({xb, xb + x.size(), "x"});
  g_bufs.push_back({codes, codes + code_bytes, "codes"});
  g_bufs.push_back({scales, scales + scale_bytes, "scales"});
  g_bufs.push_back({rotb, rotb + rot_bytes, "rot"});
  a.x = xb;
  a.row_stride = row_stride;
  a.rows = rows;
  a.codes = codes;
  a.scales = scales;
  a.rot32 = argc > 9 ? (float*)rotb : nullptr;
  a.opts = opts;
  // a small grid so that workgroups loop over rows (RBQ_EMU_GRID overrides)
  const char* g = getenv("RBQ_EMU_GRID");
  const uint32_t want = g ? (uint32_t)atoi(g) : 2u;
  const uint32_t grid = (uint32_t)(rows < want ? rows : want);
  if (in == IN_F32) run<IN_F32>(a, words, grid);
  else if (in == IN_BF16) run<IN_BF16>(a, words, grid);
  else run<IN_F16>(a, words, grid);
  write_file(argv[7], codes, code_bytes);
  write_file(argv[8], scales, scale_bytes);
  if (argc > 9) write_file(argv[9], rotb, rot_bytes);
  printf("%u %u %u %u %u\n", a.m, 1u << a.p_log, a.paley, a.q, words);
  return 0;
}
