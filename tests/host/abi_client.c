/* A plain C client of include/rbq.h: compiled by gcc, linked against librbq.so, no
 * Python and no device memory. It checks what the boundary promises without a GPU:
 * status strings, the version string, rejection of invalid arguments before any HIP
 * call, and (run with RBQ_FAULT_INJECT=launch) that every valid call reports RBQ_EHIP
 * without launching.
 *
 * Usage: abi_client validate | abi_client inject. Exit status 0 = all checks passed;
 * each failed check prints one line. */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "rbq.h"

static int failures = 0;

#define EXPECT(call, want)                                                              \
  do {                                                                                  \
    rbq_status got_ = (call);                                                           \
    if (got_ != (want)) {                                                               \
      printf("FAIL %s:%d %s -> %s, want %s\n", __FILE__, __LINE__, #call,               \
             rbq_status_string(got_), rbq_status_string(want));                         \
      ++failures;                                                                       \
    }                                                                                   \
  } while (0)

/* 16-byte aligned addresses that are never dereferenced: every call below either fails
 * validation or is stopped by the fault-injection switch before it reaches the GPU. */
#define PX ((void *)0x10000)
#define PC ((void *)0x20000)
#define PS ((void *)0x30000)

int main(int argc, char **argv) {
  const int inject = argc > 1 && strcmp(argv[1], "inject") == 0;
  if (inject) {
    /* the valid calls below pass fake addresses: without the switch that stops every
       launch they would reach the device, so refuse to run them at all */
    const char *fi = getenv("RBQ_FAULT_INJECT");
    if (!fi || strcmp(fi, "launch") != 0) {
      puts("abi_client inject: RBQ_FAULT_INJECT=launch is required (refusing to make calls that would launch)");
      return 2;
    }
  }
  const rbq_status launched = inject ? RBQ_EHIP : RBQ_OK;
  const int64_t B = 2, H = 4, S = 16, D = 128;
  const int64_t st[4] = {H * S * D, S * D, D, 1};
  const int64_t bad_st[4] = {H * S * D, S * D, D, 2};

  if (strcmp(rbq_status_string(RBQ_OK), "RBQ_OK") != 0) { puts("FAIL status string"); ++failures; }
  if (strcmp(rbq_status_string((rbq_status)42), "RBQ_UNKNOWN") != 0) { puts("FAIL unknown status"); ++failures; }
  if (!strstr(rbq_version(), "gfx950")) { puts("FAIL version"); ++failures; }

  /* empty problems succeed without launching, in both modes */
  EXPECT(hadamard_quant_int4(PX, RBQ_BF16, 4096, 0, 4096, PC, PS, RBQ_F16, NULL, RBQ_PACKED, NULL), RBQ_OK);
  EXPECT(kv_rotate_quant(PX, PX, RBQ_BF16, B, H, 0, D, st, st, PC, PS, PC, PS, RBQ_F16, NULL, 0, NULL), RBQ_OK);
  EXPECT(w4a4_gemm(PC, PS, PC, PS, RBQ_F16, 0, 64, 4096, PX, NULL, NULL), RBQ_OK);

  /* invalid arguments are rejected on the host in both modes */
  EXPECT(hadamard_quant_int4(PX, RBQ_BF16, 4095, 8, 4096, PC, PS, RBQ_F16, NULL, RBQ_PACKED, NULL), RBQ_EINVAL);
  EXPECT(hadamard_quant_int4(NULL, RBQ_BF16, 4096, 8, 4096, PC, PS, RBQ_F16, NULL, RBQ_PACKED, NULL), RBQ_EINVAL);
  EXPECT(hadamard_quant_int4_signed(PX, RBQ_BF16, 4096, 8, 4096, NULL, PC, PS, RBQ_F16, NULL, RBQ_PACKED, NULL),
         RBQ_EINVAL);
  EXPECT(hadamard_quant_int8(PX, RBQ_BF16, 4096, 8, 4096, (int8_t *)PC, PS, RBQ_F16, NULL, RBQ_PACKED, NULL),
         RBQ_EINVAL);
  EXPECT(kv_rotate_quant(PX, PX, RBQ_BF16, B, H, S, D, bad_st, st, PC, PS, PC, PS, RBQ_F16, NULL, 0, NULL),
         RBQ_EINVAL);
  EXPECT(kv_rope_rotate_quant(PX, PX, RBQ_BF16, B, H, S, D, st, st, (const float *)PS, (const float *)PS, S, 1,
                              PC, PS, PC, PS, RBQ_F16, NULL, 0, NULL),
         RBQ_EINVAL);
  EXPECT(hadamard_kron_quant_int4(PX, RBQ_BF16, 16640, 8, 16640, PC, PS, RBQ_F16, NULL, RBQ_PACKED, NULL),
         RBQ_ENOTSUP);
  EXPECT(hadamard_kron_quant_int4(PX, RBQ_BF16, 5120, 8, 5120, PC, PS, RBQ_F16, NULL, RBQ_NO_ROTATE, NULL),
         RBQ_EINVAL);
  {
    int64_t m = 0;
    EXPECT(rbq_kron_factor(14336, &m), RBQ_OK);
    if (m != 28) { printf("FAIL kron factor of 14336: %lld\n", (long long)m); ++failures; }
    EXPECT(rbq_kron_factor(11008, &m), RBQ_OK);
    if (m != 172) { printf("FAIL kron factor of 11008: %lld\n", (long long)m); ++failures; }
    EXPECT(rbq_kron_factor(16640, &m), RBQ_ENOTSUP);
    EXPECT(rbq_kron_factor(0, &m), RBQ_EINVAL);
  }
  EXPECT(quantize_groups_int4(PX, RBQ_F32, 4096, 8, 4096, 48, PC, PS, RBQ_F16, RBQ_PACKED, NULL), RBQ_EINVAL);
  EXPECT(w4a8_gemm_grouped((const int8_t *)PC, PS, PC, PS, RBQ_F16, 16, 64, 64, 4096, PX, NULL), RBQ_EINVAL);
  EXPECT(attention_decode_int4kv(PX, RBQ_BF16, PC, PS, PC, PS, RBQ_F16, 2, 8, 2, 16, 16, 64, 0.1f, PX, NULL),
         RBQ_ENOTSUP);
  EXPECT(attention_decode_int4kv(PX, RBQ_BF16, PC, PS, PC, PS, RBQ_F16, 2, 8, 3, 16, 16, 128, 0.1f, PX, NULL),
         RBQ_EINVAL);
  /* split attention: bad split counts, a short or missing workspace, head_dim 64 */
  EXPECT(attention_decode_int4kv_split(PX, RBQ_BF16, PC, PS, PC, PS, RBQ_F16, 2, 8, 2, 16, 16, 128, 0.1f, 0, PS,
                                       1 << 20, PX, NULL),
         RBQ_EINVAL);
  EXPECT(attention_decode_int4kv_split(PX, RBQ_BF16, PC, PS, PC, PS, RBQ_F16, 2, 8, 2, 16, 16, 128, 0.1f, 4097, PS,
                                       1 << 30, PX, NULL),
         RBQ_EINVAL);
  EXPECT(attention_decode_int4kv_split(PX, RBQ_BF16, PC, PS, PC, PS, RBQ_F16, 2, 8, 2, 16, 16, 128, 0.1f, 4, PS,
                                       2 * 8 * 4 * 130 * 4 - 4, PX, NULL),
         RBQ_EINVAL);
  EXPECT(attention_decode_int4kv_split(PX, RBQ_BF16, PC, PS, PC, PS, RBQ_F16, 2, 8, 2, 16, 16, 128, 0.1f, 4, NULL,
                                       1 << 20, PX, NULL),
         RBQ_EINVAL);
  EXPECT(attention_decode_int4kv_split(PX, RBQ_BF16, PC, PS, PC, PS, RBQ_F16, 2, 8, 2, 16, 16, 64, 0.1f, 4, PS,
                                       1 << 20, PX, NULL),
         RBQ_ENOTSUP);
  EXPECT(attention_decode_int4kv_split(PX, RBQ_BF16, PC, PS, PC, PS, RBQ_F16, 0, 8, 2, 16, 16, 128, 0.1f, 4, NULL,
                                       0, PX, NULL),
         RBQ_OK); /* empty batch: nothing to do, no workspace needed */
  /* the allocation-free variant: its array holds 8 MiB of partials (520 bytes per range) */
  EXPECT(attention_decode_int4kv_split_noalloc(PX, RBQ_BF16, PC, PS, PC, PS, RBQ_F16, 64, 64, 64, 16, 16, 128, 0.1f,
                                               4, PX, NULL),
         RBQ_ENOTSUP);
  EXPECT(attention_decode_int4kv_split_noalloc(PX, RBQ_BF16, PC, PS, PC, PS, RBQ_F16, 2, 8, 2, 16, 16, 128, 0.1f,
                                               0, PX, NULL),
         RBQ_EINVAL);
  EXPECT(attention_decode_int4kv_split_noalloc(PX, RBQ_BF16, PC, PS, PC, PS, RBQ_F16, 2, 8, 2, 16, 16, 64, 0.1f, 4,
                                               PX, NULL),
         RBQ_ENOTSUP);
  {
    int64_t bytes = 0;
    EXPECT(rbq_attention_split_workspace_bytes(2, 8, 4, &bytes), RBQ_OK);
    if (bytes != 2 * 8 * 4 * 130 * 4) { printf("FAIL split workspace bytes: %lld\n", (long long)bytes); ++failures; }
    EXPECT(rbq_attention_split_workspace_bytes(2, 8, 0, &bytes), RBQ_EINVAL);
    EXPECT(rbq_attention_split_workspace_bytes(2, 8, 4, NULL), RBQ_EINVAL);
  }
  EXPECT(w4a4_gemm(PC, PS, PC, PS, RBQ_F16, 64, 64, 4000, PX, NULL, NULL), RBQ_ENOTSUP);
  EXPECT(kv_cache_append_int4(PX, PX, PX, RBQ_BF16, B, H, H / 2, S, D, st, st, st, NULL, NULL, 0, 8, S + 7,
                              PS, PC, PS, PC, PS, RBQ_F16, NULL),
         RBQ_EINVAL);  /* pos0 + seq beyond the capacity */
  EXPECT(kv_cache_append_int4(PX, PX, PX, RBQ_BF16, B, H, 3, S, D, st, st, st, NULL, NULL, 0, 0, S,
                              PS, PC, PS, PC, PS, RBQ_F16, NULL),
         RBQ_EINVAL);  /* heads not a multiple of kv_heads */
  EXPECT(kv_cache_append_int4(PX, PX, PX, RBQ_BF16, B, H, H, S, 32, st, st, st, NULL, NULL, 0, 0, S,
                              PS, PC, PS, PC, PS, RBQ_F16, NULL),
         RBQ_ENOTSUP);
  EXPECT(rbq_hbm_probe(PX, 4000, PC, 4096, 8, NULL), RBQ_EINVAL);
  EXPECT(rbq_hbm_probe(PX, 0, PC, 0, 8, NULL), RBQ_EINVAL);
  EXPECT(rbq_hbm_probe(PX, 4096, NULL, 4096, 8, NULL), RBQ_EINVAL);
  EXPECT(rbq_hbm_probe(PX, 4096, PC, 4096, 0, NULL), RBQ_OK);
  EXPECT(w4a8_gemm((const int8_t *)PC, PS, PC, PS, RBQ_F16, 64, 60, 4096, PX, NULL, NULL), RBQ_ENOTSUP);

  /* valid calls: only reached in inject mode, where nothing is launched */
  if (inject) {
    EXPECT(hadamard_quant_int4(PX, RBQ_BF16, 4096, 8, 4096, PC, PS, RBQ_F16, NULL, RBQ_PACKED, NULL), launched);
    EXPECT(hadamard_quant_int4_signed(PX, RBQ_F16, 4096, 8, 4096, PS, PC, PS, RBQ_F32, NULL, RBQ_PACKED, NULL),
           launched);
    EXPECT(hadamard_quant_int8(PX, RBQ_F32, 1024, 3, 1024, (int8_t *)PC, PS, RBQ_F16, NULL, 0, NULL), launched);
    EXPECT(kv_rotate_quant(PX, PX, RBQ_BF16, B, H, S, D, st, st, PC, PS, PC, PS, RBQ_F16, NULL, 0, NULL), launched);
    EXPECT(kv_rope_rotate_quant(PX, PX, RBQ_BF16, B, H, S, D, st, st, (const float *)PS, (const float *)PS, S, 0,
                                PC, PS, PC, PS, RBQ_F16, NULL, 0, NULL),
           launched);
    EXPECT(hadamard_kron_quant_int4(PX, RBQ_BF16, 5120, 8, 5120, PC, PS, RBQ_F16, NULL, RBQ_PACKED, NULL),
           launched);
    EXPECT(quantize_groups_int4(PX, RBQ_F32, 4096, 8, 4096, 256, PC, PS, RBQ_F16, RBQ_PACKED, NULL), launched);
    EXPECT(w4a8_gemm_grouped((const int8_t *)PC, PS, PC, PS, RBQ_F16, 256, 64, 64, 4096, PX, NULL), launched);
    EXPECT(w4a8_gemm_grouped((const int8_t *)PC, PS, PC, PS, RBQ_F32, 32, 64, 64, 4096, PX, NULL), launched);
    EXPECT(attention_decode_int4kv(PX, RBQ_BF16, PC, PS, PC, PS, RBQ_F16, 2, 8, 2, 16, 16, 128, 0.1f, PX, NULL),
           launched);
    EXPECT(w4a4_gemm(PC, PS, PC, PS, RBQ_F16, 64, 64, 4096, PX, NULL, NULL), launched);
    EXPECT(w4a8_gemm((const int8_t *)PC, PS, PC, PS, RBQ_F16, 64, 64, 4096, PX, NULL, NULL), launched);
    EXPECT(rbq_hbm_probe(PX, 65536, PC, 16384, 8, NULL), launched);
    EXPECT(kv_cache_append_int4(PX, PX, PX, RBQ_BF16, B, H, H / 2, S, D, st, st, st, (const float *)PS,
                                (const float *)PS, 2 * S, 3, S + 3, PS, PC, PS, PC, PS, RBQ_F16, NULL),
           launched);
    EXPECT(attention_decode_int4kv_split(PX, RBQ_BF16, PC, PS, PC, PS, RBQ_F16, 2, 8, 2, 16, 16, 128, 0.1f, 4, PS,
                                         2 * 8 * 4 * 130 * 4, PX, NULL),
           launched);
    /* RoPE into the cache without a query: the unused query tensor stays empty */
    EXPECT(kv_cache_append_int4(NULL, PX, PX, RBQ_BF16, B, H, H / 2, S, D, st, st, st, (const float *)PS,
                                (const float *)PS, 2 * S, 3, S + 3, NULL, PC, PS, PC, PS, RBQ_F16, NULL),
           launched);
    EXPECT(attention_decode_int4kv_split_noalloc(PX, RBQ_BF16, PC, PS, PC, PS, RBQ_F16, 64, 64, 64, 16, 16, 128,
                                                 0.1f, 3, PX, NULL),
           launched);
  }

  printf("%s: %d failure(s)\n", inject ? "inject" : "validate", failures);
  return failures ? 1 : 0;
}
