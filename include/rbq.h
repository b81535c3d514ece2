/*
 * rbq.h -- C ABI of the online-rotation hot path for MI355X (gfx950).
 *
 * What it computes (all three calls, restated from the pages):
 *
 *  - A fixed Sylvester-Hadamard rotation y = H_n x / sqrt(n) per row
 *    ("Rotations: QuaRot, SpinQuant and incoherence", section "Hadamard matrices";
 *    computed as an O(n log n) fast transform per the same page's section "Why it's
 *    free: computational invariance"), fused with
 *  - per-row symmetric INT4 absmax quantization: scale s = max(max|y| / 7, 1e-8)
 *    stored in the scale dtype (round to nearest even), codes
 *    q = round_half_even(clamp(y / s_stored, -8, 7))
 *    ("SpinQuant Guide: Learned Rotations for 4-Bit LLMs", outlier-curse figure,
 *    step-size equation and the uniform_quantize_int4 listing), packed two per byte
 *    (element 2j in the low nibble, element 2j+1 in the high nibble, two's complement);
 *  - R3: the same op per (batch, head, token) vector of post-RoPE Q and K over head_dim
 *    ("SpinQuant, when rotations are worth learning", section "Four rotation sites");
 *  - the W4A4 GEMM that consumes packed codes: out[m,n] = sA[m] sW[n] sum_k qA[m,k] qW[n,k]
 *    ("SpinQuant: rotate before you round", section "Deployment implications";
 *    "SpinQuant Guide...", section "The Orthogonal Invariance Principle").
 *
 * Conventions shared by every call:
 *  - Every pointer argument is a DEVICE pointer owned by the caller; the library never
 *    allocates, frees or synchronizes, keeps no global state and is thread-safe.
 *  - Work is enqueued asynchronously on `stream` (NULL = the default stream).
 *  - Arguments are validated on the host before any HIP call. On a non-OK status
 *    nothing is launched and no output is written.
 *  - Inputs must be finite; NaN/Inf inputs are outside the contract.
 *  - Sizes are element counts unless stated otherwise.
 *
 * Diagnostics, read once per process from the environment:
 *  - RBQ_LOG=1: every call that passes validation prints one line to stderr with its
 *    sizes and the kernel variant and grid it launches.
 *  - RBQ_FAULT_INJECT=launch: every call that passes validation returns RBQ_EHIP
 *    without launching anything, so callers can test their error handling (also on a
 *    machine without a GPU).
 */
#ifndef RBQ_H
#define RBQ_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  RBQ_OK = 0,      /* success (also for an empty problem, which launches nothing) */
  RBQ_EINVAL = 1,  /* invalid argument: NULL pointer, bad size, misalignment, bad dtype */
  RBQ_ENOTSUP = 2, /* valid but unsupported combination (e.g. K % 128 != 0 in the GEMM) */
  RBQ_EHIP = 3     /* the HIP launch failed (hipGetLastError after the launch) */
} rbq_status;

typedef enum { RBQ_F32 = 0, RBQ_BF16 = 1, RBQ_F16 = 2 } rbq_dtype;

enum {
  RBQ_PACKED = 1u << 0,        /* codes two per byte; otherwise one int8 per element */
  RBQ_NO_ROTATE = 1u << 1,     /* quantize x itself (no Hadamard, no 1/sqrt(n)) */
  RBQ_Q_ROTATE_ONLY = 1u << 2  /* kv_rotate_quant: write Q rotated (bf16), do not quantize Q */
};

/*
 * hadamard_quant_int4 -- rotate each of `tokens` rows of length n by H_n / sqrt(n)
 * (natural Sylvester order), then quantize each row to INT4 with one absmax scale.
 * This is the R4 path (down-projection input) and the offline weight rotation
 * (rows of W rotated along K, which equals W H^T / sqrt(K) because H is symmetric).
 *
 *  x            [tokens, n] row-major with row stride `x_row_stride` (elements, >= n),
 *               dtype x_dtype (F32, BF16, F16). The start of every row must be aligned
 *               to min(16, n * element size) bytes.
 *  n            power of two, 2 <= n <= 32768 (the pages' K-cache path likewise
 *               requires a power-of-two size for the fast transform).
 *  tokens       number of rows, >= 0; 0 returns RBQ_OK without launching.
 *  codes        RBQ_PACKED: uint8 [tokens, n/2], contiguous; else int8 [tokens, n].
 *               16-byte aligned.
 *  scales       [tokens] contiguous, scale_dtype F32 or F16 (stored scale s_stored).
 *               Rows whose stored scale is 0 (fp16 underflow) get all-zero codes.
 *  rotated      optional float [tokens, n] contiguous, 16-byte aligned: y = H x / sqrt(n)
 *               as computed (or x itself with RBQ_NO_ROTATE); NULL skips it.
 *  flags        RBQ_PACKED, RBQ_NO_ROTATE.
 * Errors: RBQ_EINVAL for NULL x/codes/scales (when tokens > 0), n not a power of two
 * in [2, 32768], tokens < 0, x_row_stride < n, misaligned pointers/strides, a bad dtype
 * or unknown flag bits; RBQ_EHIP if the launch fails.
 */
rbq_status hadamard_quant_int4(const void *x, rbq_dtype x_dtype, int64_t n, int64_t tokens,
                               int64_t x_row_stride, void *codes, void *scales,
                               rbq_dtype scale_dtype, float *rotated, unsigned flags,
                               hipStream_t stream);

/*
 * hadamard_quant_int4_signed -- as hadamard_quant_int4 with the randomized transform
 * H_n diag(signs) / sqrt(n) ("Rotations: QuaRot, SpinQuant and incoherence", section
 * "Hadamard matrices": a random +-1 diagonal before the normalised Hadamard makes the
 * largest entry close to the row's RMS with high probability).
 *
 *  signs        device vector [n] of +1 / -1 in x_dtype (any value's sign bit is used),
 *               aligned like a row of x; owned by the caller, read only. The same
 *               diagonal applies to every row; rotated (if given) holds H diag(s) x / sqrt(n).
 *  all other arguments as for hadamard_quant_int4.
 * Errors: as hadamard_quant_int4, plus RBQ_EINVAL for a NULL or misaligned `signs` (when
 * tokens > 0) or for RBQ_NO_ROTATE (the diagonal only makes sense with the rotation).
 */
rbq_status hadamard_quant_int4_signed(const void *x, rbq_dtype x_dtype, int64_t n,
                                      int64_t tokens, int64_t x_row_stride, const void *signs,
                                      void *codes, void *scales, rbq_dtype scale_dtype,
                                      float *rotated, unsigned flags, hipStream_t stream);

/*
 * hadamard_quant_int8 -- as hadamard_quant_int4 with 8-bit codes for W4A8 layers: the
 * step-size equation of "SpinQuant Guide: Learned Rotations for 4-Bit LLMs" at b = 8,
 * s = max(max|y| / 127, 1e-8) rounded to scale_dtype, q = RNE(clamp(y / s, -128, 127)).
 *
 *  codes        int8 [tokens, n] contiguous, 16-byte aligned (one code per byte).
 *  flags        RBQ_NO_ROTATE only (RBQ_PACKED is rejected).
 *  all other arguments and errors as for hadamard_quant_int4.
 */
rbq_status hadamard_quant_int8(const void *x, rbq_dtype x_dtype, int64_t n, int64_t tokens,
                               int64_t x_row_stride, int8_t *codes, void *scales,
                               rbq_dtype scale_dtype, float *rotated, unsigned flags,
                               hipStream_t stream);

/*
 * kv_rotate_quant -- R3: rotate every head_dim vector of post-RoPE Q and K by
 * H_d / sqrt(d) and quantize it to INT4 with one scale per (batch, head, token).
 * Q and K are processed in one launch.
 *
 *  q, k         [batch, heads, seq, head_dim], dtype BF16 or F16, element strides
 *               q_strides[4] / k_strides[4] in (b, h, s, d) order; the d stride must be 1
 *               and every vector start 16-byte aligned (head_dim * 2 >= 16).
 *  head_dim     power of two, 8 <= head_dim <= 32768; a layout whose vectors are not
 *               equally spaced (non-flattenable strides) needs head_dim 64, 128 or 256
 *               (else RBQ_ENOTSUP).
 *  q_codes, k_codes   uint8 [batch, heads, seq, head_dim/2] contiguous, 16-byte aligned.
 *  q_scales, k_scales [batch, heads, seq] contiguous, scale_dtype (F16 or F32).
 *  q_rotated    with RBQ_Q_ROTATE_ONLY: bf16/f16 (same dtype as q) [batch, heads, seq,
 *               head_dim] contiguous, receives H q / sqrt(d) rounded to nearest even;
 *               q_codes and q_scales are then not written and may be NULL.
 *  flags        RBQ_Q_ROTATE_ONLY (codes are always packed two per byte).
 * Errors: RBQ_EINVAL for NULL required pointers, non-positive/inconsistent sizes,
 * head_dim not a power of two in range, a d stride != 1, misalignment, bad dtypes or
 * flags; an empty problem (any of batch, heads, seq == 0) returns RBQ_OK.
 */
rbq_status kv_rotate_quant(const void *q, const void *k, rbq_dtype dtype, int64_t batch,
                           int64_t heads, int64_t seq, int64_t head_dim,
                           const int64_t q_strides[4], const int64_t k_strides[4],
                           uint8_t *q_codes, void *q_scales, uint8_t *k_codes, void *k_scales,
                           rbq_dtype scale_dtype, void *q_rotated, unsigned flags,
                           hipStream_t stream);

/*
 * kv_rope_rotate_quant -- kv_rotate_quant with the rotary position embedding applied first,
 * so pre-RoPE Q and K go straight to KV4 codes ("SpinQuant, when rotations are worth
 * learning", section "Four rotation sites": R3 acts on queries and keys after RoPE;
 * "SpinQuant Guide: Learned Rotations for 4-Bit LLMs": RoPE turns coordinate pairs by
 * position-dependent angles). Element i pairs with i + D/2 (i < D/2); at position
 * p = rope_pos0 + s (s = the token index of the vector):
 *     x'[i] = x[i] cos[p][i] - x[i + D/2] sin[p][i],
 *     x'[i + D/2] = x[i + D/2] cos[p][i] + x[i] sin[p][i],
 * evaluated in fp32 (each product and the sum rounded, no fused multiply-add) and rounded
 * to the input's 16-bit format (nearest even) -- the values an unfused RoPE would store --
 * then rotated by H_D / sqrt(D) and quantized as by kv_rotate_quant.
 *
 *  rope_cos, rope_sin  device fp32 [rope_positions, head_dim / 2] row-major, 16-byte
 *               aligned, owned by the caller, read only.
 *  rope_positions  rows of the tables; rope_pos0 + seq must not exceed it.
 *  rope_pos0    position of token 0 (>= 0), e.g. the cache length when appending.
 *  head_dim     64, 128 or 256 (other sizes return RBQ_ENOTSUP).
 *  all other arguments as for kv_rotate_quant (RBQ_Q_ROTATE_ONLY writes RoPE'd and
 *  rotated Q in bf16/fp16).
 * Errors: as kv_rotate_quant, plus RBQ_EINVAL for NULL or misaligned tables, a negative
 * rope_pos0 or tables that do not cover the positions; RBQ_ENOTSUP for head_dim other
 * than 64, 128 and 256.
 */
rbq_status kv_rope_rotate_quant(const void *q, const void *k, rbq_dtype dtype, int64_t batch,
                                int64_t heads, int64_t seq, int64_t head_dim,
                                const int64_t q_strides[4], const int64_t k_strides[4],
                                const float *rope_cos, const float *rope_sin,
                                int64_t rope_positions, int64_t rope_pos0, uint8_t *q_codes,
                                void *q_scales, uint8_t *k_codes, void *k_scales,
                                rbq_dtype scale_dtype, void *q_rotated, unsigned flags,
                                hipStream_t stream);

/*
 * kv_cache_append_int4 -- one attention step's writes to the KV4 cache: RoPE, then the R3
 * rotation H_D / sqrt(D), then INT4 for the keys, written straight into the cache at
 * positions pos0 .. pos0 + seq - 1 ("SpinQuant, when rotations are worth learning",
 * section "Four rotation sites": R3 follows RoPE so that the KV cache can be quantized;
 * "SpinQuant Guide: Learned Rotations for 4-Bit LLMs", the transformer-block figure: keys
 * stored in the KV cache as INT4). Values are quantized to INT4 per (batch, head, token)
 * without a rotation (their rotation R2 is folded offline into the weights) and appended
 * the same way; queries get RoPE and R3 and are written in the input's 16-bit format, the
 * operand attention_decode_int4kv takes. RoPE and the quantizer are those of
 * kv_rope_rotate_quant and kv_rotate_quant (codes two per byte, low nibble first, one scale
 * per (batch, head, token)); keys and values of tokens outside the written positions are
 * left as they are. Two launches on `stream` (queries and keys, then values).
 *
 *  q            optional [batch, heads, seq, head_dim] (NULL: no query output), element
 *               strides q_strides[4] in (b, h, s, d) order, d stride 1, vectors 16-byte
 *               aligned; dtype BF16 or F16 (k and v the same).
 *  k, v         [batch, kv_heads, seq, head_dim], strides k_strides[4] / v_strides[4] as for q.
 *  heads        query heads, a multiple of kv_heads (grouped heads share a key/value head).
 *  head_dim     64, 128 or 256 (other powers of two: RBQ_ENOTSUP).
 *  rope_cos, rope_sin  optional fp32 [rope_positions, head_dim / 2] tables as for
 *               kv_rope_rotate_quant (both NULL: queries and keys are taken as already
 *               rotated by RoPE); token s of this call sits at position pos0 + s.
 *  pos0         first cache position written (>= 0), the number of tokens already cached.
 *  seq_cap      cache capacity per (batch, kv head); pos0 + seq <= seq_cap.
 *  q_rotated    with q: [batch, heads, seq, head_dim] contiguous, 16-byte aligned, in q's dtype:
 *               H RoPE(q) / sqrt(D) rounded to nearest even.
 *  k_cache, v_cache  uint8 [batch, kv_heads, seq_cap, head_dim / 2] contiguous, 16-byte aligned.
 *  k_cache_scales, v_cache_scales  [batch, kv_heads, seq_cap] contiguous in scale_dtype (F16 or F32).
 * Errors: RBQ_EINVAL for NULL required pointers (q and q_rotated go together), bad dtypes,
 * negative sizes, heads not a multiple of kv_heads, pos0 + seq > seq_cap, a d stride != 1,
 * misalignment, one RoPE table without the other or tables that do not cover the positions;
 * RBQ_ENOTSUP for head_dim other than 64, 128 and 256; an empty problem (batch, kv_heads or
 * seq == 0) returns RBQ_OK; RBQ_EHIP if a launch fails.
 */
rbq_status kv_cache_append_int4(const void *q, const void *k, const void *v, rbq_dtype dtype,
                                int64_t batch, int64_t heads, int64_t kv_heads, int64_t seq,
                                int64_t head_dim, const int64_t q_strides[4],
                                const int64_t k_strides[4], const int64_t v_strides[4],
                                const float *rope_cos, const float *rope_sin,
                                int64_t rope_positions, int64_t pos0, int64_t seq_cap,
                                void *q_rotated, uint8_t *k_cache, void *k_cache_scales,
                                uint8_t *v_cache, void *v_cache_scales, rbq_dtype scale_dtype,
                                hipStream_t stream);

/*
 * w4a4_gemm -- out[m, n] = bf16( sA[m] * sW[n] * sum_k qA[m, k] * qW[n, k] ).
 * Codes are the packed INT4 produced above (two per byte, low nibble = even k).
 * The integer sum is exact (int32 accumulation on int8 matrix cores).
 *
 *  qA     uint8 [M, K/2] row-major (K-contiguous), 16-byte aligned.
 *  sA     [M] scale_dtype (F16 or F32).
 *  qW     uint8 [N, K/2] row-major (K-contiguous), 16-byte aligned.
 *  sW     [N] scale_dtype.
 *  out_bf16  bf16 [M, N] row-major, 16-byte aligned (round to nearest even).
 *  acc    optional int32 [M, N] row-major: the exact integer sums; NULL skips it.
 *  M, N   >= 0 (0 returns RBQ_OK); K > 0, K % 128 == 0 and K <= 65536 (else
 *         RBQ_ENOTSUP: the int32 sums of 16x-scaled int8 products stay exact below that);
 *         N % 8 == 0 (else RBQ_ENOTSUP).
 * Errors: RBQ_EINVAL for NULL pointers, negative sizes, odd K, misalignment or a bad
 * scale dtype; RBQ_ENOTSUP as above; RBQ_EHIP if the launch fails.
 */
rbq_status w4a4_gemm(const uint8_t *qA, const void *sA, const uint8_t *qW, const void *sW,
                     rbq_dtype scale_dtype, int64_t M, int64_t N, int64_t K, void *out_bf16,
                     int32_t *acc, hipStream_t stream);

/*
 * w4a8_gemm -- the W4A8 variant: INT8 activation codes (hadamard_quant_int8) times packed
 * INT4 weight codes, out[m, n] = bf16( sA[m] * sW[n] * sum_k qA[m, k] * qW[n, k] ). The
 * pages' only latency figure is for this configuration ("SpinQuant: LLM Quantization with
 * Learned Rotations", measured effects); the step-size equation of "SpinQuant Guide:
 * Learned Rotations for 4-Bit LLMs" at b = 8 gives the activation codes.
 *
 *  qA     int8 [M, K] row-major (K-contiguous), 16-byte aligned.
 *  qW     uint8 [N, K/2] packed INT4 as for w4a4_gemm.
 *  all other arguments, limits (K % 128 == 0, K <= 65536, N % 8 == 0) and errors as for
 *  w4a4_gemm; the integer sums are exact.
 */
rbq_status w4a8_gemm(const int8_t *qA, const void *sA, const uint8_t *qW, const void *sW,
                     rbq_dtype scale_dtype, int64_t M, int64_t N, int64_t K, void *out_bf16,
                     int32_t *acc, hipStream_t stream);

/*
 * attention_decode_int4kv -- decode attention of one query position per (batch, head) over
 * the INT4 key/value cache: keys as kv_rotate_quant writes them (R3-rotated, packed INT4,
 * one scale per token and head), values as hadamard_quant_int4 writes them with
 * RBQ_NO_ROTATE per (token, head) row. Because the query is rotated by the same
 * orthogonal H / sqrt(head_dim) as the keys, the scores equal those of the unrotated pair
 * ("SpinQuant, when rotations are worth learning", section "Four rotation sites"):
 *   score[s] = softmax_scale * sum_d q[d] * k_scale[s] * k_code[s, d]
 *   out[d]   = sum_s softmax(score)[s] * v_scale[s] * v_code[s, d]
 * with key/value head kvh = h / (heads / kv_heads). Arithmetic in fp32; the output is
 * rounded to the query's format. With 2 or more query heads per key/value head (an even
 * number of them) and at least 256 workgroups' worth of (batch, key/value head, set of 2 or
 * 4 query heads), one workgroup reads each cached token once for its set of query heads;
 * otherwise one workgroup per (batch, query head). The two orders round differently (both
 * within the fp32 error the parity tests bound).
 *
 *  q         [batch, heads, head_dim] contiguous, BF16 or F16 (kv_rotate_quant's rotated Q
 *            with RBQ_Q_ROTATE_ONLY), 16-byte aligned.
 *  k_codes, v_codes  uint8 [batch, kv_heads, seq_cap, head_dim/2], 16-byte aligned; tokens
 *            0 .. seq-1 of each head are used (seq_cap is the cache capacity).
 *  k_scales, v_scales  [batch, kv_heads, seq_cap] in scale_dtype (F16 or F32).
 *  head_dim  128 (others: RBQ_ENOTSUP).
 *  out       [batch, heads, head_dim] in q_dtype, 16-byte aligned.
 * Errors: RBQ_EINVAL for NULL or misaligned pointers, bad dtypes, seq < 1, seq_cap < seq,
 * heads not a multiple of kv_heads or a NaN scale; RBQ_ENOTSUP for head_dim != 128,
 * seq >= 2^26 (one head's codes are addressed with 32-bit byte offsets), seq_cap > 2^30
 * or (batch + 8) * heads > 2^31 - 1 (the grid is padded to whole groups of 8 key/value heads).
 */
rbq_status attention_decode_int4kv(const void *q, rbq_dtype q_dtype, const uint8_t *k_codes,
                                   const void *k_scales, const uint8_t *v_codes,
                                   const void *v_scales, rbq_dtype scale_dtype, int64_t batch,
                                   int64_t heads, int64_t kv_heads, int64_t seq, int64_t seq_cap,
                                   int64_t head_dim, float softmax_scale, void *out,
                                   hipStream_t stream);

/*
 * attention_decode_int4kv_split -- attention_decode_int4kv with each (batch, head)'s tokens
 * cut into `splits` ranges of ceil(seq / splits) tokens, one workgroup per range, so that
 * few (batch, head) pairs still fill the device. Each range's workgroup writes its partial
 * maximum m, sum l and unnormalised output o (fp32, [batch * heads, splits, 2 + 128]) to
 * `workspace`; a second kernel on the same stream combines the ranges in order,
 *   out[d] = sum_r e^(m_r - M) o_r[d] / sum_r e^(m_r - M) l_r,  M = max_r m_r,
 * the softmax of attention_decode_int4kv summed in another grouping (the same real value;
 * fp32 rounding differs). The attention itself is the one the pages define for K and V
 * cached in INT4; the split is a scheduling choice of this library, not theirs.
 *
 *  all arguments as attention_decode_int4kv, plus:
 *  splits           1 .. 4096; ranges past the sequence's end contribute nothing.
 *  workspace        device memory of at least workspace_bytes, 16-byte aligned, owned by the
 *                   caller; not read before it is written; free for reuse once the call's
 *                   kernels have finished on `stream`.
 *  workspace_bytes  at least rbq_attention_split_workspace_bytes(batch, heads, splits).
 * Errors: as attention_decode_int4kv, plus RBQ_EINVAL for splits outside 1 .. 4096 or a
 * NULL, misaligned or short workspace; RBQ_ENOTSUP when batch * heads * splits + 8 * heads > 2^31 - 1.
 */
rbq_status attention_decode_int4kv_split(const void *q, rbq_dtype q_dtype, const uint8_t *k_codes,
                                         const void *k_scales, const uint8_t *v_codes,
                                         const void *v_scales, rbq_dtype scale_dtype, int64_t batch,
                                         int64_t heads, int64_t kv_heads, int64_t seq, int64_t seq_cap,
                                         int64_t head_dim, float softmax_scale, int64_t splits,
                                         void *workspace, int64_t workspace_bytes, void *out,
                                         hipStream_t stream);

/*
 * rbq_attention_split_workspace_bytes -- the workspace attention_decode_int4kv_split needs:
 * batch * heads * splits * 130 * 4 bytes, written to *bytes. RBQ_EINVAL for a NULL `bytes`,
 * negative sizes or splits outside 1 .. 4096; RBQ_ENOTSUP if batch * heads > 2^31 - 1.
 */
rbq_status rbq_attention_split_workspace_bytes(int64_t batch, int64_t heads, int64_t splits, int64_t *bytes);

/*
 * attention_decode_int4kv_split_noalloc -- attention_decode_int4kv_split for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the ranges' partials go to a fixed array of 8 MiB that
 * the library holds on each GPU it runs on until the process ends, so the call takes no
 * workspace and allocates nothing. Its device address is looked up once per device (with
 * that device current), on the first call there.
 *
 *  all other arguments as attention_decode_int4kv_split.
 *  limit   batch * heads * splits * 130 * 4 <= 8 MiB (else RBQ_ENOTSUP, nothing launched).
 * The array keeps the last call's partials; nothing in it needs to start at zero. Calls
 * that overlap on one GPU (other streams, other threads) share the array and race: the
 * caller serialises them. Errors: as attention_decode_int4kv_split, plus RBQ_ENOTSUP above
 * the limit and RBQ_EHIP if the array's address cannot be found.
 */
rbq_status attention_decode_int4kv_split_noalloc(const void *q, rbq_dtype q_dtype, const uint8_t *k_codes,
                                                 const void *k_scales, const uint8_t *v_codes,
                                                 const void *v_scales, rbq_dtype scale_dtype, int64_t batch,
                                                 int64_t heads, int64_t kv_heads, int64_t seq,
                                                 int64_t seq_cap, int64_t head_dim, float softmax_scale,
                                                 int64_t splits, void *out, hipStream_t stream);

/*
 * w4a8_gemm_grouped -- W4A8 with group-wise weight scales: one scale per run of `group`
 * consecutive K elements of each weight row ("SpinQuant, when rotations are worth
 * learning": its ExecuTorch export uses 4-bit weights in groups of 256 or 32 input
 * channels with 8-bit dynamic activations):
 *   out[m, n] = bf16( sA[m] * sum_g sW[n, g] * sum_{k in group g} qA[m, k] * qW[n, k] ),
 * each group's integer sum exact, the scaled group sums added in fp32.
 *
 *  qA     int8 [M, K] (hadamard_quant_int8 codes), 16-byte aligned.
 *  qW     uint8 [N, K/2] packed INT4 (quantize_groups_int4 codes), 16-byte aligned.
 *  sA     [M]; sW [N, K/group] row-major; both scale_dtype (F16 or F32).
 *  group  power of two, 32 <= group <= K, dividing K.
 *  out_bf16 bf16 [M, N] row-major, 16-byte aligned.
 * Errors: as w4a4_gemm, plus RBQ_EINVAL for a bad group size.
 */
rbq_status w4a8_gemm_grouped(const int8_t *qA, const void *sA, const uint8_t *qW, const void *sW,
                             rbq_dtype scale_dtype, int64_t group, int64_t M, int64_t N,
                             int64_t K, void *out_bf16, hipStream_t stream);

/*
 * quantize_groups_int4 -- group-wise symmetric INT4 quantization of rows that are already
 * in the rotated basis (the offline weight path: rows rotated by hadamard_quant_int4's
 * `rotated` output, then quantized per group): each run of `group` consecutive elements
 * gets s = max(max|y_g| / 7, 1e-8), stored in scale_dtype, and codes
 * round_half_even(clamp(y / s_stored, -8, 7)) ("SpinQuant Guide: Learned Rotations for
 * 4-Bit LLMs", step-size equation, per group).
 *
 *  y        [rows, K], dtype F32, BF16 or F16, row stride `y_row_stride` elements; rows
 *           16-byte aligned.
 *  group    power of two, 32 <= group <= min(K, 4096), dividing K.
 *  codes    RBQ_PACKED: uint8 [rows, K/2]; else int8 [rows, K]; 16-byte aligned.
 *  scales   [rows, K/group] row-major in scale_dtype (F32 or F16).
 *  flags    RBQ_PACKED only.
 * Errors: RBQ_EINVAL for NULL pointers (rows > 0), misalignment, a bad dtype, group size or
 * flag; RBQ_EHIP if the launch fails.
 */
rbq_status quantize_groups_int4(const void *y, rbq_dtype dtype, int64_t K, int64_t rows,
                                int64_t y_row_stride, int64_t group, void *codes, void *scales,
                                rbq_dtype scale_dtype, unsigned flags, hipStream_t stream);

/*
 * hadamard_kron_quant_int4 -- hadamard_quant_int4 for row lengths that are not powers of
 * two ("Rotations: QuaRot, SpinQuant and incoherence", section "Hadamard matrices": such
 * lengths use the Kronecker product of a power-of-two Hadamard matrix with a small known
 * one). n = m * p with p a power of two, and each row is rotated by
 * (H_m (x) H_p) / sqrt(n), element a * p + b of the row being index (a, b) of the
 * product; H_p is the Sylvester matrix and H_m one of:
 *   Paley I (q = m - 1 prime, q = 3 mod 4): I + [[0, 1...], [-1..., Q]],
 *     Q[a][b] = chi(a - b) with chi the quadratic character of GF(q);
 *   Paley II (q = m/2 - 1 prime, q = 1 mod 4): the conference matrix [[0, 1...], [1..., Q]]
 *     with each 0 replaced by [[1, -1], [-1, -1]] and each +-1 by +-[[1, 1], [1, -1]];
 *   m = 172: the Goethals-Seidel array [[A, BR, CR, DR], [-BR, A, D^T R, -C^T R],
 *     [-CR, -D^T R, A, B^T R], [-DR, C^T R, -B^T R, A]] (R the back-diagonal permutation)
 *     of circulant +-1 matrices A, B, C, D of order 43 whose periodic autocorrelations
 *     add up to zero at every nonzero shift; their first rows are constant on the cosets
 *     of the order-7 subgroup of (Z/43)^* and are the lexicographically first such
 *     quadruple (+1 at 0 for bit 0 of a code, +1 on the j-th coset for bit j, cosets by
 *     smallest element). This covers the FFN width 11008 = 172 * 64.
 * m is the smallest of 4o, 8o, 16o, ... (o the odd part of n, m <= 256, m dividing n) with
 * one of these constructions (rbq_kron_factor reports it). The quantizer, the codes and
 * the scales are those of hadamard_quant_int4.
 *
 *  x, x_dtype, tokens, x_row_stride, codes, scales, scale_dtype, rotated: as for
 *               hadamard_quant_int4; x rows 16-byte aligned.
 *  n            2 <= n <= 32768. A power of two is passed to hadamard_quant_int4.
 *  flags        RBQ_PACKED only.
 * Errors: RBQ_EINVAL for the argument errors of hadamard_quant_int4 and for flags other
 * than RBQ_PACKED; RBQ_ENOTSUP when n has no factor by the rule above or the kernel does
 * not take it (p < 16, p > 2048, or the [m, p] row buffer and the m x m operand table
 * exceed 160 KiB of LDS, e.g. 172 * 128); RBQ_EHIP if the launch fails.
 */
rbq_status hadamard_kron_quant_int4(const void *x, rbq_dtype x_dtype, int64_t n, int64_t tokens,
                                    int64_t x_row_stride, void *codes, void *scales,
                                    rbq_dtype scale_dtype, float *rotated, unsigned flags,
                                    hipStream_t stream);

/*
 * rbq_kron_factor -- the order m of the small factor hadamard_kron_quant_int4 uses for a
 * row length n (1 for a power of two). Host only, no HIP call.
 * Errors: RBQ_EINVAL for n < 1 or m == NULL; RBQ_ENOTSUP when the rule finds no factor.
 */
rbq_status rbq_kron_factor(int64_t n, int64_t *m);

/*
 * rbq_hbm_probe -- measurement only, not part of the method: a streaming kernel shaped
 * like the row kernels above, whose rate is the ceiling this device reaches for a given
 * mix of HBM reads and writes (the published 8 TB/s is the other reference). Workgroup b
 * reads bytes [b * read_bytes_per_block, (b + 1) * read_bytes_per_block) of src with
 * 16-byte loads, then writes bytes [b * write_bytes_per_block, ...) of dst with a value
 * derived from what it read.
 *
 *  src      device buffer of blocks * read_bytes_per_block bytes (may be NULL when
 *           read_bytes_per_block is 0), 16-byte aligned, read only.
 *  dst      device buffer of blocks * write_bytes_per_block bytes, 16-byte aligned; with
 *           write_bytes_per_block == 0 it must hold 16 * blocks bytes, of which a
 *           workgroup writes one word only when its folded loads equal 0x9E3779B9.
 *  read_bytes_per_block, write_bytes_per_block  multiples of 4096, not both 0.
 *  blocks   number of workgroups (0 returns RBQ_OK).
 * Errors: RBQ_EINVAL for NULL or misaligned buffers, negative sizes or sizes that are not
 * multiples of 4096; RBQ_EHIP if the launch fails.
 */
rbq_status rbq_hbm_probe(const void *src, int64_t read_bytes_per_block, void *dst,
                         int64_t write_bytes_per_block, int64_t blocks, hipStream_t stream);

/* Human-readable name of a status code (static string, never NULL). */
const char *rbq_status_string(rbq_status s);

/* Library version string (static). */
const char *rbq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RBQ_H */
