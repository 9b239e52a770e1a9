/*
 * tbq4.h -- C ABI of libtbq4: flash attention read directly from a TBQ4 KV
 * cache on AMD Instinct MI355X (gfx950).
 *
 * Source of the method: the page "Kontekst 262K na jednej RTX 4090: co
 * dodałem do llama.cpp-turboq" (trefon.com notes).
 *   - section "Od czego zacząłem": a TBQ4 block stores 128 values in 66 bytes,
 *     a 2-byte scale followed by 64 bytes of 4-bit indices (4.125 bits per
 *     value); the flash-attention kernel reads raw TBQ4 blocks from global
 *     memory and dequantises them in its inner loop; attention works in the
 *     rotated (Hadamard) domain, so there is no separate dequantisation pass
 *     and no F16 buffer.
 *   - section "Konfiguracja": the K and the V cache each get their own type
 *     (-ctk tbq4_0 -ctv tbq4_0); flash attention on; the context length is
 *     fixed up front (-c 262144).
 *   - section "4. Poprawność w długich sesjach": a full context must be
 *     handled gracefully rather than crash -- here every capacity overflow is
 *     an error code returned before anything is launched.
 *
 * Block format (one block = one head vector of one token, head_dim 128):
 *   u = R x with R = H D / sqrt(128): D = diag(s), s in {+1,-1}^128 drawn from
 *   SplitMix64(sign_seed) (bit i of the two 64-bit outputs, little endian,
 *   set means s_i = -1), H the natural-order Sylvester Hadamard matrix.
 *   bytes 0-1   d = binary16 nearest sqrt(mean(u_i^2)), ties to even,
 *               saturating at 65504, little endian
 *   bytes 2-65  4-bit codes, element 2j in the low nibble of byte 2+j and
 *               element 2j+1 in the high nibble.  A code is sign-magnitude
 *               (laid out like the e2m1 4-bit float): bit 3 set for u_i < 0,
 *               bits 0-2 = m_i = number of midpoints tau_k of adjacent
 *               magnitudes with d*tau_k < |u_i| (nearest level, ties toward
 *               zero, u_i = 0 -> +0.125).
 *   magnitudes  0.125 0.375 0.625 0.9375 1.25 1.625 2 2.75  (tau_k = midpoints)
 *   Dequantised value in the rotated domain: d * (-1)^sign * magnitude[m];
 *   x_hat = R^T (d c).
 *
 * Conventions shared by every call
 *   - Every pointer argument named as device memory is caller-owned device
 *     memory; the library never allocates, frees or caches device memory and
 *     keeps no mutable global state (calls are re-entrant and thread-safe).
 *     The one exception is tbq4_attn_decode_noalloc, for callers that cannot
 *     allocate: it uses a static device array that the library holds per
 *     device (see its declaration).
 *   - All work is enqueued on `hip_stream` (a hipStream_t; NULL = the null
 *     stream).  No call synchronises.  Order appends before attention on the
 *     same stream.
 *   - Every argument check runs on the host before any launch; a failing
 *     call returns a negative status and touches no memory.  A launch failure
 *     reported by the HIP runtime returns TBQ4_ERR_HIP.
 *   - Non-finite inputs give undefined (but memory-safe) results.
 */
#ifndef TBQ4_H
#define TBQ4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TBQ4_HEAD_DIM 128
#define TBQ4_BLOCK_BYTES 66
#define TBQ4_MAX_SPLITS 1024

typedef enum {
  TBQ4_OK = 0,
  TBQ4_ERR_INVALID_ARG = -1, /* null pointer, bad count, bad dtype, ...   */
  TBQ4_ERR_UNSUPPORTED = -2, /* head_dim != 128, n_q_heads % n_kv_heads   */
  TBQ4_ERR_CAPACITY = -3,    /* a token range runs past the capacity      */
  TBQ4_ERR_ALIGNMENT = -4,   /* pointer not 16-byte aligned, capacity % 8 */
  TBQ4_ERR_WORKSPACE = -5,   /* workspace missing or too small            */
  TBQ4_ERR_HIP = -6          /* the HIP runtime reported a launch error   */
} tbq4_status;

typedef enum { TBQ4_F32 = 0, TBQ4_F16 = 1, TBQ4_BF16 = 2 } tbq4_dtype;

/* One layer's K and V caches.
 *   k, v        device memory, caller-owned, layout [batch][n_kv_heads]
 *               [capacity][66] bytes each (tbq4_cache_bytes() bytes), 16-byte
 *               aligned.  Blocks are position independent, so a caller can
 *               checkpoint or copy any byte range.
 *   head_dim    must be 128.
 *   capacity    tokens per sequence; a multiple of 8 (keeps every head's
 *               row of blocks 16-byte aligned).
 *   sign_seed   seeds the sign vector shared by K, V, Q and the output. */
typedef struct {
  uint8_t *k;
  uint8_t *v;
  int32_t batch;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t capacity;
  uint64_t sign_seed;
} tbq4_cache;

/* Bytes of ONE of the two caches: batch * n_kv_heads * capacity * 66.
 * Returns 0 for a negative argument. */
size_t tbq4_cache_bytes(int32_t batch, int32_t n_kv_heads, int32_t capacity);

/* Split count tbq4_attn_decode uses when given n_splits = 0 (depends only on
 * the shapes), so callers can size the workspace.  Returns 0 on bad input. */
int32_t tbq4_decode_auto_splits(int32_t batch, int32_t n_kv_heads, int32_t n_ctx);

/* Workspace bytes tbq4_attn_decode needs for `n_splits` splits (n_splits = 0
 * means the automatic count for these shapes):
 * batch * n_q_heads * n_splits * 130 * 4 (fp32 max, sum and 128 partial
 * outputs per split), rounded up to 256.  Returns 0 on bad input. */
size_t tbq4_decode_workspace_bytes(int32_t batch, int32_t n_kv_heads, int32_t n_q_heads,
                                   int32_t n_ctx, int32_t n_splits);

/* The 16 bytes of the sign vector for `seed` (host memory, caller-owned):
 * the first two SplitMix64 outputs, little endian. */
tbq4_status tbq4_sign_vector(uint64_t seed, uint8_t out_bits[16]);

/* Quantise and append new K and V rows (the write side of the cache).
 * Page "Kontekst 262K na jednej RTX 4090: co dodałem do llama.cpp-turboq",
 * section "Od czego zacząłem": each head vector becomes one 66-byte TBQ4
 * block (2-byte scale, 64 bytes of 4-bit indices) in the rotated Hadamard
 * domain; section "Konfiguracja" fixes the cache size up front (-c), which is
 * why writes past the capacity are an error, not a reallocation.
 *   k_new, v_new  device, [batch][n_new][n_kv_heads][128] in src_dtype,
 *                 16-byte aligned.
 *   Writes the blocks of token slots [pos, pos + n_new) of every sequence of
 *   both caches; other slots are untouched.  pos >= 0 and pos + n_new <=
 *   capacity, else TBQ4_ERR_CAPACITY.  n_new = 0 is a no-op.
 *   The packed bytes are a pure function of the input values and sign_seed
 *   (fp64 arithmetic throughout). */
tbq4_status tbq4_quantize_append(const tbq4_cache *cache, const void *k_new,
                                 const void *v_new, tbq4_dtype src_dtype,
                                 int32_t pos, int32_t n_new, void *hip_stream);

/* Quantise a flat array of n_blocks blocks of 128 values (device, src_dtype)
 * into n_blocks * 66 bytes at `out` (device).  Same arithmetic as
 * tbq4_quantize_append; for callers that keep their own cache layout. */
tbq4_status tbq4_quantize_blocks(const void *x, tbq4_dtype src_dtype, int64_t n_blocks,
                                 uint64_t sign_seed, uint8_t *out, void *hip_stream);

/* Decode attention: one query per (sequence, query head) against cached
 * slots [0, n_ctx) of its KV head (kv head = h / (n_q_heads / n_kv_heads)).
 * Page "Kontekst 262K na jednej RTX 4090: co dodałem do llama.cpp-turboq",
 * section "Od czego zacząłem": flash attention reads the raw TBQ4 blocks and
 * dequantises them in its inner loop, in the rotated domain, with no
 * dequantisation pass and no F16 buffer; the result is softmax attention
 * over the dequantised cache.
 *   q            device, [batch][n_q_heads][128], q_dtype (F32, F16 or BF16)
 *   out          device, [batch][n_q_heads][128], out_dtype (F16 or F32)
 *   softmax_scale multiplies q.k before the softmax
 *   n_splits     split-K partition count in [1, 1024], or 0 for automatic
 *   workspace    device, >= tbq4_decode_workspace_bytes(...) bytes, 16-byte
 *                aligned; scratch for the per-split partial softmax states.
 * Errors: 1 <= n_ctx <= capacity else TBQ4_ERR_CAPACITY; n_q_heads a positive
 * multiple of n_kv_heads with n_q_heads / n_kv_heads <= 8, else
 * TBQ4_ERR_UNSUPPORTED.  Two launches (split kernel, merge kernel). */
tbq4_status tbq4_attn_decode(const tbq4_cache *cache, const void *q, tbq4_dtype q_dtype,
                             int32_t n_q_heads, int32_t n_ctx, float softmax_scale,
                             void *out, tbq4_dtype out_dtype, int32_t n_splits,
                             void *workspace, size_t workspace_bytes, void *hip_stream);

/* Decode attention that allocates nothing and takes no workspace: for
 * callers that cannot allocate device memory or pass a scratch buffer (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments, checks, kernels and results as
 * tbq4_attn_decode minus the workspace: the split-K partial states go to a
 * static device array of TBQ4_NOALLOC_SCRATCH_BYTES that the library holds
 * on every device it runs on until the process ends.
 *   - Calls whose partial states exceed the array (batch * n_q_heads *
 *     n_splits * 520 bytes, rounded up to 256, with n_splits the automatic
 *     count when 0 is given) return TBQ4_ERR_WORKSPACE before any HIP call.
 *   - The array's device address is looked up (hipGetSymbolAddress) on the
 *     first call on each device; make that first call outside graph capture.
 *   - All calls on one device share that device's array: calls that overlap
 *     on one device (different streams, or different threads) race.  Calls
 *     ordered on one stream do not.  Nothing in the array needs to start at
 *     zero; the previous call's contents are simply overwritten.
 * Calls no hipMalloc, hipFree or allocating library routine. */
#define TBQ4_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
tbq4_status tbq4_attn_decode_noalloc(const tbq4_cache *cache, const void *q, tbq4_dtype q_dtype,
                                     int32_t n_q_heads, int32_t n_ctx, float softmax_scale,
                                     void *out, tbq4_dtype out_dtype, int32_t n_splits,
                                     void *hip_stream);

/* The two phases of tbq4_attn_decode, for callers that produce or combine
 * split-K partial states themselves (for example partials computed over
 * different token ranges, or on different devices, then merged).
 *
 * tbq4_attn_decode_partial: same arguments and checks as tbq4_attn_decode
 * minus the output; writes, for every (sequence b, query head h, split p),
 * 130 fp32 values at workspace + ((b * n_q_heads + h) * n_splits + p) * 130:
 *   [0] m  = the split's reference score, in log2 units (softmax_scale *
 *          log2(e) * q.k): one of its scores, at most 8 below the split's
 *          maximum (max - 8 <= m <= max; the kernel moves it only when a
 *          score exceeds it by more than 8); -inf for an empty split
 *   [1] l  = sum over the split's keys of 2^(score - m)
 *   [2 + i] = sum over the split's keys of 2^(score - m) * v'_i, i = 0..127,
 *          in the ROTATED domain (v' = R v, unnormalised).
 * Split p covers the 32-token tiles [p * T, (p + 1) * T), T = ceil(ceil(n_ctx
 * / 32) / n_splits); with n_splits = 0 the automatic count is used and
 * returned through *n_splits_used (may be NULL).
 *
 * tbq4_attn_decode_merge: out[b][h] = R^T (sum_p 2^(m_p - M) o_p / sum_p
 * 2^(m_p - M) l_p), M = max_p m_p, from a workspace laid out as above with
 * n_splits partial states per (b, h).  sign_seed must be the cache's. */
tbq4_status tbq4_attn_decode_partial(const tbq4_cache *cache, const void *q, tbq4_dtype q_dtype,
                                     int32_t n_q_heads, int32_t n_ctx, float softmax_scale,
                                     int32_t n_splits, int32_t *n_splits_used, void *workspace,
                                     size_t workspace_bytes, void *hip_stream);
/* tbq4_attn_decode_partial_timed: tbq4_attn_decode_partial plus two optional
 * HIP events (hipEvent_t, created by the caller with timing enabled; either
 * may be NULL).  The split kernel's own dispatch records them at the start and
 * at the end of its execution, so hipEventElapsedTime on the pair gives the
 * kernel's duration without the latency of separate event markers.  For
 * callers that time the kernel in production without a profiler. */
tbq4_status tbq4_attn_decode_partial_timed(const tbq4_cache *cache, const void *q,
                                           tbq4_dtype q_dtype, int32_t n_q_heads, int32_t n_ctx,
                                           float softmax_scale, int32_t n_splits,
                                           int32_t *n_splits_used, void *workspace,
                                           size_t workspace_bytes, void *hip_stream,
                                           void *start_event, void *stop_event);
tbq4_status tbq4_attn_decode_merge(const void *workspace, size_t workspace_bytes, int32_t batch,
                                   int32_t n_q_heads, int32_t n_splits, uint64_t sign_seed,
                                   void *out, tbq4_dtype out_dtype, void *hip_stream);

/* Mixed K/V cache formats.
 *
 * Page "Kontekst 262K na jednej RTX 4090: co dodałem do llama.cpp-turboq",
 * section "Konfiguracja": the K and the V cache types are chosen separately
 * (-ctk, -ctv).  The DFlash speed-test page (gptunnel blog), section "Қосымша
 * олжа: кванттталған KV-кэш жылдамдықтың 39%-ын жейді", measures what a
 * quantised cache costs against an fp16 one.  These calls let each tensor be
 * TBQ4 or TBQ3 blocks, q8_0 rows or plain fp16 rows, so the dequantisation
 * cost can be weighed against the bytes saved per tensor.
 *
 *   TBQ4_FMT_TBQ4  66-byte blocks as above, rotated by the cache's signs
 *   TBQ4_FMT_F16   head vectors stored as 128 binary16 values (round to
 *                  nearest even from the input, overflow to infinity), not
 *                  rotated: 256 bytes per head vector
 *   TBQ4_FMT_TBQ3  50-byte blocks, the 3-bit sibling of TBQ4 (same page,
 *                  section "6. Ten sam cache na Apple silicon", which runs a
 *                  TBQ3 cache beside TBQ4 and fixes its 3-bit packing).  The
 *                  page gives no codebook, so this library reads it as: the
 *                  same rotation and binary16 scale d as TBQ4, then per
 *                  rotated value the nearest of +-d x {0.25, 0.75, 1.375,
 *                  2.25} (the 8-level Gaussian quantiser restricted to four
 *                  significant bits; ties go to the smaller magnitude), code
 *                  = magnitude index | 4 if negative; code i sits at bits
 *                  3i .. 3i+2 of the little-endian integer held in bytes
 *                  2 .. 49.  3.125 bits per value.
 *   TBQ4_FMT_Q8_0  136-byte rows, not rotated: four blocks of 32 values,
 *                  each the binary16 scale d (little endian) then 32 int8
 *                  codes (34 bytes).  The pages name q8_0 as a KV cache type
 *                  (the tgstat.ru channel @tech_di page's server
 *                  configuration sets both tensors to it) without defining
 *                  it; read as: d32 = max|x| / 127 and q = x / d32 in IEEE
 *                  fp32, q rounded to the nearest integer with halves away
 *                  from zero, d = the binary16 nearest d32.  8.5 bits per
 *                  value.  Inputs must be finite.
 * tbq4_mixed_cache: k, v point at [batch][n_kv_heads][capacity][row bytes of
 * their format] (tbq4_format_row_bytes), 16-byte aligned; the rest as in
 * tbq4_cache, capacity a multiple of 8.  Unknown formats are
 * TBQ4_ERR_UNSUPPORTED.
 * tbq4_mixed_append: as tbq4_quantize_append, each tensor in its format.
 * tbq4_mixed_attn_decode: as tbq4_attn_decode (same workspace size, G <= 8):
 *   q is rotated only when K is stored rotated (TBQ4 or TBQ3), and the
 *   output is rotated back only when V is.  Any combination of the four
 *   formats is accepted. */
typedef enum { TBQ4_FMT_TBQ4 = 0, TBQ4_FMT_F16 = 1, TBQ4_FMT_TBQ3 = 2, TBQ4_FMT_Q8_0 = 3 } tbq4_format;
typedef struct {
  uint8_t *k;
  uint8_t *v;
  int32_t k_format;
  int32_t v_format;
  int32_t batch;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t capacity;
  uint64_t sign_seed;
} tbq4_mixed_cache;
size_t tbq4_format_row_bytes(int32_t format);
tbq4_status tbq4_mixed_append(const tbq4_mixed_cache *cache, const void *k_new, const void *v_new,
                              tbq4_dtype src_dtype, int32_t pos, int32_t n_new, void *hip_stream);
tbq4_status tbq4_mixed_attn_decode(const tbq4_mixed_cache *cache, const void *q,
                                   tbq4_dtype q_dtype, int32_t n_q_heads, int32_t n_ctx,
                                   float softmax_scale, void *out, tbq4_dtype out_dtype,
                                   int32_t n_splits, void *workspace, size_t workspace_bytes,
                                   void *hip_stream);

/* Multi-query verify attention (the current token plus up to three drafted
 * ones, per sequence).
 *
 * Page "Kontekst 262K na jednej RTX 4090: co dodałem do llama.cpp-turboq":
 * its production decode runs multi-token prediction (--spec-type mtp
 * --spec-draft-n-max 3), so every step verifies 1 + up to 3 drafted tokens
 * against the cache; section "Od czego zacząłem" gives the attention itself.
 * Query i (0 <= i < n_q <= 4) of sequence b sits at absolute position
 * n_past + i and attends slots [0, n_past + i]: causal among the new tokens,
 * full over the prefix.  Slots [n_past, n_past + n_q) must already hold the
 * new tokens' K and V (tbq4_quantize_append first), as for prefill.
 *   q, out    device [batch][n_q][n_q_heads][128] (q fp32/fp16/bf16, out
 *             fp32/fp16), 16-byte aligned
 *   n_splits  split-K count in [1, 1024] or 0 for automatic; workspace of
 *             tbq4_verify_workspace_bytes(..., n_splits) bytes, 16-byte
 *             aligned, laid out as the decode workspace with row index
 *             b * n_q + i in place of b
 * Every (query, head) is computed from one pass over the cache: the K and V
 * tiles are dequantised once for all n_q queries.  G = n_q_heads /
 * n_kv_heads <= 8.  Two launches (split kernel, decode merge kernel).
 * Errors: n_q outside [1, 4] or G > 8 -> TBQ4_ERR_UNSUPPORTED;
 * n_past + n_q > capacity -> TBQ4_ERR_CAPACITY; otherwise as tbq4_attn_decode. */
size_t tbq4_verify_workspace_bytes(int32_t batch, int32_t n_kv_heads, int32_t n_q_heads,
                                   int32_t n_past, int32_t n_q, int32_t n_splits);
tbq4_status tbq4_attn_verify(const tbq4_cache *cache, const void *q, tbq4_dtype q_dtype,
                             int32_t n_q_heads, int32_t n_past, int32_t n_q, float softmax_scale,
                             void *out, tbq4_dtype out_dtype, int32_t n_splits, void *workspace,
                             size_t workspace_bytes, void *hip_stream);

/* Device-side lengths (ragged batches) and graph-stable decode.
 *
 * Page "Kontekst 262K na jednej RTX 4090: co dodałem do llama.cpp-turboq",
 * section "2. Mniej przechwyceń grafu CUDA": padding the KV length to a
 * coarse minimum cuts how often the decode graph must be re-captured as the
 * context grows.  These two calls go further: the launch shapes depend only
 * on (batch, heads, max_ctx, n_splits), and every per-step value -- where
 * each sequence appends, how many slots each sequence attends -- is read
 * from device memory, so one captured HIP graph of "append, then attend"
 * replays unchanged while the lengths advance on the device.
 *
 * tbq4_quantize_append_at: as tbq4_quantize_append, but sequence b writes
 *   slots [positions[b], positions[b] + n_new).  positions: device int32
 *   [batch], read when the kernel runs.  Slots outside [0, capacity) are
 *   skipped (the positions cannot be checked on the host); n_new must not
 *   exceed capacity (TBQ4_ERR_CAPACITY).
 * tbq4_attn_decode_varlen: as tbq4_attn_decode, but sequence b attends slots
 *   [0, ctx_lens[b]).  ctx_lens: device int32 [batch], each clamped to
 *   [0, max_ctx]; 1 <= max_ctx <= capacity (TBQ4_ERR_CAPACITY otherwise).
 *   n_splits = 0 and the workspace size follow max_ctx
 *   (tbq4_decode_workspace_bytes with n_ctx = max_ctx).  Each sequence's
 *   slots are spread evenly over the n_splits splits at its own length.  A
 *   sequence of length 0 gets a zero output. */
tbq4_status tbq4_quantize_append_at(const tbq4_cache *cache, const void *k_new, const void *v_new,
                                    tbq4_dtype src_dtype, const int32_t *positions, int32_t n_new,
                                    void *hip_stream);
tbq4_status tbq4_attn_decode_varlen(const tbq4_cache *cache, const void *q, tbq4_dtype q_dtype,
                                    int32_t n_q_heads, const int32_t *ctx_lens, int32_t max_ctx,
                                    float softmax_scale, void *out, tbq4_dtype out_dtype,
                                    int32_t n_splits, void *workspace, size_t workspace_bytes,
                                    void *hip_stream);

/* Decode step: append one token per sequence and attend over the cache that
 * now holds it, in two launches instead of three.  The one-token step of a
 * generation loop (page "Kontekst 262K na jednej RTX 4090: co dodałem do
 * llama.cpp-turboq", section "Od czego zacząłem": quantise the new K/V into
 * the cache, then flash attention over the raw blocks).  Same results as
 * tbq4_quantize_append(k_new, v_new, pos, n_new = 1) followed by
 * tbq4_attn_decode(n_ctx = pos + 1): the stored bytes are identical; the
 * output differs only in rounding (the new token's score and value are
 * taken in fp64 from its codes instead of through the fp16 MFMA operands).
 * In the decode launch one extra wavefront per (sequence, KV head)
 * quantises and stores the token and writes its own partial softmax state,
 * while the other wavefronts stream the slots before it.
 *   k_new, v_new  device, [batch][1][n_kv_heads][128] in src_dtype (F32, F16
 *                 or BF16), 16-byte aligned.
 *   pos, positions  positions == NULL: every sequence writes slot pos and
 *                 attends slots [0, pos]; 0 <= pos < capacity, else
 *                 TBQ4_ERR_CAPACITY.  positions = device int32 [batch], read
 *                 when the kernel runs: sequence b writes slot positions[b] and
 *                 attends [0, positions[b]], and pos is the largest position the
 *                 call may meet (it sets the launch shape, the automatic split
 *                 count and the workspace size, so a captured HIP graph replays
 *                 unchanged while positions advance); a position outside
 *                 [0, pos] writes nothing and gives that sequence a zero output.
 *   q, out, softmax_scale, out_dtype  as tbq4_attn_decode.
 *   n_splits     splits over the slots before the new token, in [1, 1023],
 *                or 0 for the automatic count of tbq4_attn_decode at n_ctx =
 *                pos + 1.
 *   workspace    device, >= tbq4_decode_step_workspace_bytes(batch,
 *                n_kv_heads, n_q_heads, pos + 1, n_splits) bytes, 16-byte
 *                aligned: the decode layout with n_splits + 1 partial states
 *                per (sequence, head), the new token's last.
 * Errors as tbq4_quantize_append and tbq4_attn_decode. */
size_t tbq4_decode_step_workspace_bytes(int32_t batch, int32_t n_kv_heads, int32_t n_q_heads,
                                        int32_t n_ctx, int32_t n_splits);
tbq4_status tbq4_decode_step(const tbq4_cache *cache, const void *k_new, const void *v_new,
                             tbq4_dtype src_dtype, int32_t pos, const int32_t *positions,
                             const void *q, tbq4_dtype q_dtype, int32_t n_q_heads,
                             float softmax_scale, void *out, tbq4_dtype out_dtype,
                             int32_t n_splits, void *workspace, size_t workspace_bytes,
                             void *hip_stream);
/* tbq4_decode_step_timed: tbq4_decode_step plus two optional HIP events
 * (hipEvent_t, created by the caller with timing enabled; either may be
 * NULL) that the split kernel's own dispatch records at its start and end,
 * as tbq4_attn_decode_partial_timed does: the duration of the step's main
 * kernel without a profiler. */
tbq4_status tbq4_decode_step_timed(const tbq4_cache *cache, const void *k_new, const void *v_new,
                                   tbq4_dtype src_dtype, int32_t pos, const int32_t *positions,
                                   const void *q, tbq4_dtype q_dtype, int32_t n_q_heads,
                                   float softmax_scale, void *out, tbq4_dtype out_dtype,
                                   int32_t n_splits, void *workspace, size_t workspace_bytes,
                                   void *hip_stream, void *start_event, void *stop_event);

/* Prefill-chunk attention: n_q new queries per sequence; query i sits at
 * absolute position n_past + i and attends slots [0, n_past + i] (causal
 * inside the chunk, full over the cached prefix).  Same attention as
 * tbq4_attn_decode (page "Kontekst 262K na jednej RTX 4090: co dodałem do
 * llama.cpp-turboq", section "Od czego zacząłem"), for a long prompt taken
 * in pieces (section "1. Checkpointy blokowały prefill": a 262K prefill with
 * the prompt state saved at 32 points along the way).  Slots [n_past, n_past +
 * n_q) must already hold the chunk's own K/V (tbq4_quantize_append first).
 *   q, out   device, [batch][n_q][n_q_heads][128]; q_dtype F32, F16 or BF16,
 *            out_dtype F16 or F32.
 * Range: each entry of softmax_scale * log2(e) * (R q) (R q for a K stored
 * unrotated) must stay below 2^28 in magnitude (scores far beyond any
 * meaningful softmax); larger entries may overflow to inf.
 * Errors: n_past >= 0, n_q >= 1, n_past + n_q <= capacity else
 * TBQ4_ERR_CAPACITY; n_q_heads / n_kv_heads must be 1, 2, 4, 8, 16 or 32,
 * else TBQ4_ERR_UNSUPPORTED. */
tbq4_status tbq4_attn_prefill_chunk(const tbq4_cache *cache, const void *q, tbq4_dtype q_dtype,
                                    int32_t n_q_heads, int32_t n_past, int32_t n_q,
                                    float softmax_scale, void *out, tbq4_dtype out_dtype,
                                    void *hip_stream);

/* Prefill-chunk attention on a mixed-format cache (section "6. Ten sam cache
 * na Apple silicon" runs the same attention over a TBQ3 cache; section
 * "Konfiguracja" chooses the K and V types separately): as
 * tbq4_attn_prefill_chunk, with K and V each stored as TBQ4, TBQ3, q8_0 or
 * fp16 rows (tbq4_mixed_cache; the q8_0 cache of the tgstat.ru channel
 * @tech_di page's server configuration).  q is rotated only when K is stored
 * rotated (TBQ4 or TBQ3), the output rotated back only when V is.  Errors as
 * tbq4_attn_prefill_chunk. */
tbq4_status tbq4_mixed_attn_prefill_chunk(const tbq4_mixed_cache *cache, const void *q,
                                          tbq4_dtype q_dtype, int32_t n_q_heads, int32_t n_past,
                                          int32_t n_q, float softmax_scale, void *out,
                                          tbq4_dtype out_dtype, void *hip_stream);

/* Multi-query verify attention on a mixed-format cache (the drafted-token
 * verify of page "Kontekst 262K na jednej RTX 4090: co dodałem do
 * llama.cpp-turboq" over the per-tensor types of its section "Konfiguracja"
 * and the TBQ3 cache of section "6. Ten sam cache na Apple silicon"): as
 * tbq4_attn_verify, with K and V each stored as TBQ4, TBQ3, q8_0 or fp16
 * rows (tbq4_mixed_cache).  q is rotated only when K is stored rotated, the
 * output rotated back only when V is.  The workspace size is
 * tbq4_verify_workspace_bytes as for TBQ4.  Errors as tbq4_attn_verify. */
tbq4_status tbq4_mixed_attn_verify(const tbq4_mixed_cache *cache, const void *q,
                                   tbq4_dtype q_dtype, int32_t n_q_heads, int32_t n_past,
                                   int32_t n_q, float softmax_scale, void *out,
                                   tbq4_dtype out_dtype, int32_t n_splits, void *workspace,
                                   size_t workspace_bytes, void *hip_stream);

/* Static description of a status code. */
const char *tbq4_status_str(tbq4_status s);

/* Library version as "major.minor.patch". */
const char *tbq4_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TBQ4_H */
