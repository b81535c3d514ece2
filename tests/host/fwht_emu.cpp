// Host execution of the fused Hadamard + INT4 quantizer's workgroup body (the same
// template code the HIP kernel runs), one std::thread per GPU lane, with LDS, workgroup
// barriers, wave-level synchronisation and lane shuffles emulated, and every global and
// LDS access bounds-checked. Used by tests/test_host_emulator.py to validate the data
// layouts and index arithmetic on the CPU before anything runs on a GPU.
//
// usage: fwht_emu K IN ROT FOURD rows opts mode0 x.bin x_elems row_stride
//                 codes.bin scales.bin [B H S sb sh ss]
// environment: RBQ_EMU_GRID, RBQ_EMU_FAST, RBQ_EMU_SIGNS, RBQ_EMU_ROPE, RBQ_EMU_CACHE
// (the rotated output, when requested by mode0, is written to codes.bin + ".rot")
#include <barrier>
#include <cstdio>
#include <cstdlib>
#include <memory>
#include <string>
#include <thread>
#include <vector>

#include "../../rotation_bit_quantization_fwht_amd/csrc/fwht_engine.h"
#include "host_ctx.h"

using namespace rbq;

// workgroups run one after another; with fewer workgroups than blocks each one loops
// over several blocks, as on the GPU
template <int K, int IN, bool ROT, bool FOURD>
static void run(const KArgs& a, uint32_t grid) {
  constexpr const Plan& P = PlanOf<K, use_matrix_plan(K, IN, ROT)>::value;
  const int nthreads = 64 << P.w;
  for (uint32_t wg = 0; wg < grid; ++wg) {
    WgShared sh(lds_words(P) + (1u << P.w) + 1, nthreads, 1 << P.w);
    std::vector<std::thread> th;
    for (int t = 0; t < nthreads; ++t)
      th.emplace_back([&, t] {
        HostCtx c{(uint32_t)(t & 63), (uint32_t)(t >> 6), &sh};
        const bool fast = getenv("RBQ_EMU_FAST") != nullptr;
        const bool rope = a.t[0].rope_cos != nullptr;
        if constexpr (K >= 6 && K <= 8 && IN != IN_F32) {
          if constexpr (FOURD) {
            if (a.t[0].out_cap != 0u) {  // the per-head cache output (kv_cache_append_int4)
              if constexpr (ROT) {
                if (rope) fwht_quant_persistent<K, IN, ROT, FOURD, false, true, true>(c, a, wg, grid);
                else fwht_quant_persistent<K, IN, ROT, FOURD, false, false, true>(c, a, wg, grid);
              } else {
                fwht_quant_persistent<K, IN, ROT, FOURD, false, false, true>(c, a, wg, grid);
              }
              return;
            }
          }
          if constexpr (ROT) {
            if (rope) {
              if (fast) fwht_quant_persistent<K, IN, ROT, FOURD, true, true, false>(c, a, wg, grid);
              else fwht_quant_persistent<K, IN, ROT, FOURD, false, true, false>(c, a, wg, grid);
              return;
            }
          }
        }
        if (fast) fwht_quant_persistent<K, IN, ROT, FOURD, true, false, false>(c, a, wg, grid);
        else fwht_quant_persistent<K, IN, ROT, FOURD, false, false, false>(c, a, wg, grid);
      });
    for (auto& x : th) x.join();
  }
}

template <int K>
static void run_k(const KArgs& a, uint32_t grid, int in, bool rot, bool fourd) {
  if (fourd) {
    if (in == IN_BF16) { if (rot) run<K, IN_BF16, true, true>(a, grid); else run<K, IN_BF16, false, true>(a, grid); }
    else { if (rot) run<K, IN_F16, true, true>(a, grid); else run<K, IN_F16, false, true>(a, grid); }
    return;
  }
  if (in == IN_F32) { if (rot) run<K, IN_F32, true, false>(a, grid); else run<K, IN_F32, false, false>(a, grid); }
  else if (in == IN_BF16) { if (rot) run<K, IN_BF16, true, false>(a, grid); else run<K, IN_BF16, false, false>(a, grid); }
  else { if (rot) run<K, IN_F16, true, false>(a, grid); else run<K, IN_F16, false, false>(a, grid); }
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
  if (argc < 13) { fprintf(stderr, "bad args\n"); return 2; }
  const int K = atoi(argv[1]), in = atoi(argv[2]), fourd = atoi(argv[4]);
  int rot = atoi(argv[3]);
  const long long rows = atoll(argv[5]);
  const unsigned opts = (unsigned)atoi(argv[6]), mode0 = (unsigned)atoi(argv[7]);
  std::vector<char> x = read_file(argv[8]);
  const long long row_stride = atoll(argv[10]);
  const long long n = 1ll << K;
  const int esz = in == IN_F32 ? 4 : 2;
  // 16-byte aligned copies with exact-size registration (bounds checks are tight)
  auto alloc = [](size_t bytes) { return (char*)aligned_alloc(64, ((bytes + 63) / 64) * 64 + 64); };
  char* xb = alloc(x.size());
  memcpy(xb, x.data(), x.size());
  // RBQ_EMU_CACHE="cap pos0": codes and scales go to a cache of cap rows per (batch, head)
  // at positions pos0 .. pos0 + S - 1 (needs the B H S arguments)
  long long cache_cap = 0, cache_pos0 = 0, out_rows = rows;
  if (const char* cp = getenv("RBQ_EMU_CACHE")) {
    if (sscanf(cp, "%lld %lld", &cache_cap, &cache_pos0) != 2 || argc < 19) { fprintf(stderr, "bad RBQ_EMU_CACHE\n"); return 2; }
    out_rows = atoll(argv[13]) * atoll(argv[14]) * cache_cap;
  }
  const size_t code_row = (size_t)((opts & OPT_PACKED) ? n / 2 : n), scale_size = (opts & OPT_SCALE_F16) ? 2 : 4;
  const size_t code_bytes = (size_t)out_rows * code_row;
  const size_t scale_bytes = (size_t)out_rows * scale_size;
  const size_t rot_bytes = (size_t)rows * n * ((mode0 & MODE_ROT16) ? 2 : 4);
  char* codes = alloc(code_bytes);
  char* scales = alloc(scale_bytes);
  char* rotb = alloc(rot_bytes);
  memset(codes, 0xEE, code_bytes); memset(scales, 0xEE, scale_bytes); memset(rotb, 0xEE, rot_bytes);
  g_bufs.push_back({xb, xb + x.size(), "x"});
  g_bufs.push_back({codes, codes + code_bytes, "codes"});
  g_bufs.push_back({scales, scales + scale_bytes, "scales"});
  g_bufs.push_back({rotb, rotb + rot_bytes, "rot"});
  KArgs a{};
  TensorArgs& t = a.t[0];
  t.x = xb;
  t.row_stride = row_stride;
  t.codes = codes; t.scales = scales;
  t.rot32 = (mode0 & MODE_ROT32) ? (float*)rotb : nullptr;
  t.rot16 = (mode0 & MODE_ROT16) ? (uint16_t*)rotb : nullptr;
  t.mode = mode0;
  // RBQ_EMU_SIGNS names a file with the +-1 diagonal of the randomized transform
  static std::vector<char> signs;
  if (const char* sp = getenv("RBQ_EMU_SIGNS")) {
    signs = read_file(sp);
    g_bufs.push_back({signs.data(), signs.data() + signs.size(), "signs"});
    t.signs = signs.data();
  }
  // RBQ_EMU_ROPE="cos.bin sin.bin pos0": RoPE tables (fp32 [positions, n/2])
  static std::vector<char> rope_c, rope_s;
  if (const char* rp = getenv("RBQ_EMU_ROPE")) {
    char cpath[512], spath[512];
    unsigned pos0 = 0;
    if (sscanf(rp, "%511s %511s %u", cpath, spath, &pos0) != 3) { fprintf(stderr, "bad RBQ_EMU_ROPE\n"); return 2; }
    rope_c = read_file(cpath);
    rope_s = read_file(spath);
    g_bufs.push_back({rope_c.data(), rope_c.data() + rope_c.size(), "rope_cos"});
    g_bufs.push_back({rope_s.data(), rope_s.data() + rope_s.size(), "rope_sin"});
    t.rope_cos = (const float*)rope_c.data();
    t.rope_sin = (const float*)rope_s.data();
    t.rope_pos0 = pos0;
  }
  if (argc >= 19) {
    const long long B = atoll(argv[13]), H = atoll(argv[14]), S = atoll(argv[15]);
    t.sb = atoll(argv[16]); t.sh = atoll(argv[17]); t.ss = atoll(argv[18]);
    t.seq = (uint32_t)S; t.heads = (uint32_t)H;
    t.div_s = make_fastdiv((uint32_t)S); t.div_h = make_fastdiv((uint32_t)H);
    (void)B;
    if (t.rope_cos) set_rope_order_rt(t, K);  // as the library does for RoPE launches
  }
  if (cache_cap) {
    t.out_cap = (uint32_t)cache_cap;
    t.codes = codes + cache_pos0 * code_row;
    t.scales = scales + cache_pos0 * scale_size;
  }
  t.rows = rows;
  a.t[1] = t;
  const int rl = make_plan(K, use_matrix_plan(K, in, rot != 0)).r;
  uint32_t nblocks = (uint32_t)((rows + (1ll << rl) - 1) >> rl);
  a.blocks0 = nblocks;
  a.blocks1 = nblocks;
  if (cache_cap && !rot) {
    // values of kv_cache_append_int4: quantized as they are by the rotating cache kernel's
    // as_is_rows blocks (n / 8 lanes per row), as the library launches them
    const long long nt = 64ll << make_plan(K, use_matrix_plan(K, in, true)).w;
    const long long per = nt / (n / 8);
    a.tv = t;
    a.t[0].rows = 0;
    a.t[1].rows = 0;
    a.blocks0 = 0;
    a.blocks1 = 0;
    nblocks = (uint32_t)((rows + per - 1) / per);
    rot = 1;
  }
  a.nblocks = nblocks;
  // a small grid so that workgroups loop over several blocks (RBQ_EMU_GRID overrides)
  const char* g = getenv("RBQ_EMU_GRID");
  const uint32_t want = g ? (uint32_t)atoi(g) : 3u;
  const uint32_t grid = nblocks < want ? nblocks : want;
  a.opts = opts;
  (void)esz;
  switch (K) {
#define RK(k) case k: run_k<k>(a, grid, in, rot != 0, fourd != 0); break;
    RK(1) RK(2) RK(3) RK(4) RK(5) RK(6) RK(7) RK(8) RK(9) RK(10) RK(11) RK(12) RK(13) RK(14) RK(15)
#undef RK
    default: return 2;
  }
  write_file(argv[11], codes, code_bytes);
  write_file(argv[12], scales, scale_bytes);
  // rotated output goes next to the codes file with suffix ".rot"
  if (mode0 & (MODE_ROT32 | MODE_ROT16)) {
    std::string p = std::string(argv[11]) + ".rot";
    write_file(p.c_str(), rotb, rot_bytes);
  }
  return 0;
}
