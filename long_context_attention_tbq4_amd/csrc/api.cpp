// C ABI of libtbq4 (declared in include/tbq4.h): argument checks on the host,
// then kernel launches on the caller's stream.  No device memory is allocated
// here and no call synchronises.
//
// Page "Kontekst 262K na jednej RTX 4090: co dodałem do llama.cpp-turboq":
// section "Konfiguracja" (K and V caches typed separately, context fixed up
// front) and section "4. Poprawność w długich sesjach" (a full context must be
// handled gracefully instead of crashing): every shape, capacity and pointer
// problem is a negative status returned before anything is enqueued.
#include <hip/hip_runtime.h>
#include <math.h>
#include <string.h>

#include "../../include/tbq4.h"
#include "tbq4_launch.h"

namespace {

// SplitMix64 (Steele, Lea and Flood, OOPSLA 2014): state += golden gamma,
// then two xor-shift-multiply rounds and a final xor-shift.
uint64_t splitmix64_next(uint64_t &state) {
  state += 0x9E3779B97F4A7C15ull;
  uint64_t z = state;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

void sign_words(uint64_t seed, uint32_t out[4]) {
  uint64_t st = seed;
  const uint64_t w0 = splitmix64_next(st);
  const uint64_t w1 = splitmix64_next(st);
  out[0] = (uint32_t)w0;
  out[1] = (uint32_t)(w0 >> 32);
  out[2] = (uint32_t)w1;
  out[3] = (uint32_t)(w1 >> 32);
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

tbq4_status check_cache(const tbq4_cache *c) {
  if (!c) return TBQ4_ERR_INVALID_ARG;
  if (!c->k || !c->v) return TBQ4_ERR_INVALID_ARG;
  if (c->batch <= 0 || c->n_kv_heads <= 0 || c->capacity <= 0) return TBQ4_ERR_INVALID_ARG;
  if (c->head_dim != TBQ4_HEAD_DIM) return TBQ4_ERR_UNSUPPORTED;
  if (c->capacity % 8 != 0) return TBQ4_ERR_ALIGNMENT;
  // one (sequence, head) row must stay addressable with 32-bit offsets
  if ((int64_t)c->capacity * TBQ4_BLOCK_BYTES > 0x7FFFFFF0ll) return TBQ4_ERR_UNSUPPORTED;
  if (!aligned16(c->k) || !aligned16(c->v)) return TBQ4_ERR_ALIGNMENT;
  return TBQ4_OK;
}

bool valid_dtype(int d) { return d == TBQ4_F32 || d == TBQ4_F16 || d == TBQ4_BF16; }

tbq4_status from_hip(hipError_t e) { return e == hipSuccess ? TBQ4_OK : TBQ4_ERR_HIP; }

int32_t auto_splits(int32_t batch, int32_t n_kv_heads, int32_t n_ctx) {
  // enough wavefronts for ~8 per compute unit on a 256-CU part, but never
  // fewer than 4 tiles per split
  const int64_t n_tiles = (n_ctx + tbq4::kDecodeTile - 1) / tbq4::kDecodeTile;
  const int64_t rows = (int64_t)batch * n_kv_heads;
  int64_t p = (2048 + rows - 1) / rows;
  const int64_t max_by_len = (n_tiles + 3) / 4;
  if (p > max_by_len) p = max_by_len;
  if (p < 1) p = 1;
  if (p > TBQ4_MAX_SPLITS) p = TBQ4_MAX_SPLITS;
  return (int32_t)p;
}

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

extern "C" {

size_t tbq4_cache_bytes(int32_t batch, int32_t n_kv_heads, int32_t capacity) {
  if (batch < 0 || n_kv_heads < 0 || capacity < 0) return 0;
  return (size_t)batch * (size_t)n_kv_heads * (size_t)capacity * TBQ4_BLOCK_BYTES;
}

int32_t tbq4_decode_auto_splits(int32_t batch, int32_t n_kv_heads, int32_t n_ctx) {
  if (batch <= 0 || n_kv_heads <= 0 || n_ctx <= 0) return 0;
  return auto_splits(batch, n_kv_heads, n_ctx);
}

size_t tbq4_decode_workspace_bytes(int32_t batch, int32_t n_kv_heads, int32_t n_q_heads,
                                   int32_t n_ctx, int32_t n_splits) {
  if (batch <= 0 || n_kv_heads <= 0 || n_q_heads <= 0 || n_ctx <= 0) return 0;
  if (n_splits < 0 || n_splits > TBQ4_MAX_SPLITS) return 0;
  const int32_t p = n_splits == 0 ? auto_splits(batch, n_kv_heads, n_ctx) : n_splits;
  return round256((size_t)batch * n_q_heads * p * 130 * sizeof(float));
}

tbq4_status tbq4_sign_vector(uint64_t seed, uint8_t out_bits[16]) {
  if (!out_bits) return TBQ4_ERR_INVALID_ARG;
  uint32_t w[4];
  sign_words(seed, w);
  for (int i = 0; i < 4; ++i)
    for (int j = 0; j < 4; ++j) out_bits[4 * i + j] = (uint8_t)(w[i] >> (8 * j));
  return TBQ4_OK;
}

tbq4_status tbq4_quantize_append(const tbq4_cache *cache, const void *k_new, const void *v_new,
                                 tbq4_dtype src_dtype, int32_t pos, int32_t n_new,
                                 void *hip_stream) {
  tbq4_status s = check_cache(cache);
  if (s != TBQ4_OK) return s;
  if (!valid_dtype(src_dtype)) return TBQ4_ERR_INVALID_ARG;
  if (n_new < 0 || pos < 0) return TBQ4_ERR_INVALID_ARG;
  if ((int64_t)pos + n_new > cache->capacity) return TBQ4_ERR_CAPACITY;
  if (n_new == 0) return TBQ4_OK;
  if (!k_new || !v_new) return TBQ4_ERR_INVALID_ARG;
  if (!aligned16(k_new) || !aligned16(v_new)) return TBQ4_ERR_ALIGNMENT;
  tbq4::QuantArgs a;
  memset(&a, 0, sizeof(a));
  a.src[0] = k_new;
  a.src[1] = v_new;
  a.dst[0] = cache->k;
  a.dst[1] = cache->v;
  a.blocks_per_tensor = (int64_t)cache->batch * n_new * cache->n_kv_heads;
  a.n_new = n_new;
  a.n_kv_heads = cache->n_kv_heads;
  a.capacity = cache->capacity;
  a.pos = pos;
  a.flat = 0;
  uint32_t w[4];
  sign_words(cache->sign_seed, w);
  a.sign_lo = w[0]; a.sign_hi = w[1]; a.sign_lo2 = w[2]; a.sign_hi2 = w[3];
  return from_hip(tbq4::launch_quantize(a, (int)src_dtype, 2, (hipStream_t)hip_stream));
}

tbq4_status tbq4_quantize_blocks(const void *x, tbq4_dtype src_dtype, int64_t n_blocks,
                                 uint64_t sign_seed, uint8_t *out, void *hip_stream) {
  if (!valid_dtype(src_dtype)) return TBQ4_ERR_INVALID_ARG;
  if (n_blocks < 0) return TBQ4_ERR_INVALID_ARG;
  if (n_blocks == 0) return TBQ4_OK;
  if (!x || !out) return TBQ4_ERR_INVALID_ARG;
  if (n_blocks > ((int64_t)1 << 36)) return TBQ4_ERR_UNSUPPORTED;
  tbq4::QuantArgs a;
  memset(&a, 0, sizeof(a));
  a.src[0] = x;
  a.dst[0] = out;
  a.blocks_per_tensor = n_blocks;
  a.flat = 1;
  uint32_t w[4];
  sign_words(sign_seed, w);
  a.sign_lo = w[0]; a.sign_hi = w[1]; a.sign_lo2 = w[2]; a.sign_hi2 = w[3];
  return from_hip(tbq4::launch_quantize(a, (int)src_dtype, 1, (hipStream_t)hip_stream));
}

// Checks shared by the decode calls; fills `a` (all but out) and returns the
// split count through *P.
static tbq4_status prepare_decode(const tbq4_cache *cache, const void *q, tbq4_dtype q_dtype,
                                  int32_t n_q_heads, int32_t n_ctx, float softmax_scale,
                                  int32_t n_splits, void *workspace, size_t workspace_bytes,
                                  tbq4::DecodeArgs &a) {
  tbq4_status s = check_cache(cache);
  if (s != TBQ4_OK) return s;
  if (!q) return TBQ4_ERR_INVALID_ARG;
  if (!valid_dtype(q_dtype)) return TBQ4_ERR_INVALID_ARG;   // fp32, fp16 or bf16
  if (!isfinite(softmax_scale)) return TBQ4_ERR_INVALID_ARG;
  if (n_q_heads <= 0 || n_q_heads % cache->n_kv_heads != 0) return TBQ4_ERR_UNSUPPORTED;
  const int32_t G = n_q_heads / cache->n_kv_heads;
  if (G > 8) return TBQ4_ERR_UNSUPPORTED;
  if (n_ctx < 1 || n_ctx > cache->capacity) return TBQ4_ERR_CAPACITY;
  if (n_splits < 0 || n_splits > TBQ4_MAX_SPLITS) return TBQ4_ERR_INVALID_ARG;
  if (cache->batch > 65535 || cache->n_kv_heads > 65535) return TBQ4_ERR_UNSUPPORTED;
  const int32_t P = n_splits == 0 ? auto_splits(cache->batch, cache->n_kv_heads, n_ctx) : n_splits;
  const size_t need = tbq4_decode_workspace_bytes(cache->batch, cache->n_kv_heads, n_q_heads,
                                                  n_ctx, P);
  if (!workspace || workspace_bytes < need) return TBQ4_ERR_WORKSPACE;
  if (!aligned16(workspace) || !aligned16(q)) return TBQ4_ERR_ALIGNMENT;
  memset(&a, 0, sizeof(a));
  a.k = cache->k;
  a.v = cache->v;
  a.q = q;
  a.ws = (float *)workspace;
  a.n_kv_heads = cache->n_kv_heads;
  a.n_q_heads = n_q_heads;
  a.group = G;
  a.capacity = cache->capacity;
  a.n_ctx = n_ctx;
  a.n_splits = P;
  a.rotate_out = 1;
  a.qscale = softmax_scale * 1.4426950408889634f;
  sign_words(cache->sign_seed, a.sign);
  return TBQ4_OK;
}

tbq4_status tbq4_attn_decode(const tbq4_cache *cache, const void *q, tbq4_dtype q_dtype,
                             int32_t n_q_heads, int32_t n_ctx, float softmax_scale, void *out,
                             tbq4_dtype out_dtype, int32_t n_splits, void *workspace,
                             size_t workspace_bytes, void *hip_stream) {
  if (!out) return TBQ4_ERR_INVALID_ARG;
  if (out_dtype != TBQ4_F32 && out_dtype != TBQ4_F16) return TBQ4_ERR_INVALID_ARG;
  tbq4::DecodeArgs a;
  tbq4_status s = prepare_decode(cache, q, q_dtype, n_q_heads, n_ctx, softmax_scale, n_splits,
                                 workspace, workspace_bytes, a);
  if (s != TBQ4_OK) return s;
  if (!aligned16(out)) return TBQ4_ERR_ALIGNMENT;
  a.out = out;
  hipStream_t st = (hipStream_t)hip_stream;
  s = from_hip(tbq4::launch_decode_partial(a, cache->batch, (int)q_dtype, st));
  if (s != TBQ4_OK) return s;
  return from_hip(tbq4::launch_decode_merge(a, cache->batch, (int)out_dtype, st));
}

static_assert(TBQ4_NOALLOC_SCRATCH_BYTES == tbq4::kDecodeScratchBytes,
              "the header states the scratch size the library holds");

tbq4_status tbq4_attn_decode_noalloc(const tbq4_cache *cache, const void *q, tbq4_dtype q_dtype,
                                     int32_t n_q_heads, int32_t n_ctx, float softmax_scale,
                                     void *out, tbq4_dtype out_dtype, int32_t n_splits,
                                     void *hip_stream) {
  if (!out) return TBQ4_ERR_INVALID_ARG;
  if (out_dtype != TBQ4_F32 && out_dtype != TBQ4_F16) return TBQ4_ERR_INVALID_ARG;
  // The checks of tbq4_attn_decode, with the scratch array standing for the
  // workspace (a non-null, aligned stand-in address of its size: it is never
  // dereferenced; the device address replaces it below).  Partial states that
  // would not fit are TBQ4_ERR_WORKSPACE, before any HIP call.
  tbq4::DecodeArgs a;
  tbq4_status s = prepare_decode(cache, q, q_dtype, n_q_heads, n_ctx, softmax_scale, n_splits,
                                 reinterpret_cast<void *>((uintptr_t)256),
                                 tbq4::kDecodeScratchBytes, a);
  if (s != TBQ4_OK) return s;
  if (!aligned16(out)) return TBQ4_ERR_ALIGNMENT;
  hipStream_t st = (hipStream_t)hip_stream;
  void *ws = nullptr;
  s = from_hip(tbq4::decode_scratch(st, &ws));
  if (s != TBQ4_OK) return s;
  a.ws = (float *)ws;
  a.out = out;
  s = from_hip(tbq4::launch_decode_partial(a, cache->batch, (int)q_dtype, st));
  if (s != TBQ4_OK) return s;
  return from_hip(tbq4::launch_decode_merge(a, cache->batch, (int)out_dtype, st));
}

tbq4_status tbq4_attn_decode_partial(const tbq4_cache *cache, const void *q, tbq4_dtype q_dtype,
                                     int32_t n_q_heads, int32_t n_ctx, float softmax_scale,
                                     int32_t n_splits, int32_t *n_splits_used, void *workspace,
                                     size_t workspace_bytes, void *hip_stream) {
  tbq4::DecodeArgs a;
  tbq4_status s = prepare_decode(cache, q, q_dtype, n_q_heads, n_ctx, softmax_scale, n_splits,
                                 workspace, workspace_bytes, a);
  if (s != TBQ4_OK) return s;
  if (n_splits_used) *n_splits_used = a.n_splits;
  return from_hip(tbq4::launch_decode_partial(a, cache->batch, (int)q_dtype,
                                              (hipStream_t)hip_stream));
}

tbq4_status tbq4_attn_decode_partial_timed(const tbq4_cache *cache, const void *q,
                                           tbq4_dtype q_dtype, int32_t n_q_heads, int32_t n_ctx,
                                           float softmax_scale, int32_t n_splits,
                                           int32_t *n_splits_used, void *workspace,
                                           size_t workspace_bytes, void *hip_stream,
                                           void *start_event, void *stop_event) {
  tbq4::DecodeArgs a;
  tbq4_status s = prepare_decode(cache, q, q_dtype, n_q_heads, n_ctx, softmax_scale, n_splits,
                                 workspace, workspace_bytes, a);
  if (s != TBQ4_OK) return s;
  if (n_splits_used) *n_splits_used = a.n_splits;
  return from_hip(tbq4::launch_decode_partial(a, cache->batch, (int)q_dtype,
                                              (hipStream_t)hip_stream, (hipEvent_t)start_event,
                                              (hipEvent_t)stop_event));
}

tbq4_status tbq4_attn_decode_merge(const void *workspace, size_t workspace_bytes, int32_t batch,
                                   int32_t n_q_heads, int32_t n_splits, uint64_t sign_seed,
                                   void *out, tbq4_dtype out_dtype, void *hip_stream) {
  if (!workspace || !out) return TBQ4_ERR_INVALID_ARG;
  if (out_dtype != TBQ4_F32 && out_dtype != TBQ4_F16) return TBQ4_ERR_INVALID_ARG;
  if (batch <= 0 || n_q_heads <= 0 || batch > 65535 || n_q_heads > 65535)
    return TBQ4_ERR_INVALID_ARG;
  if (n_splits < 1 || n_splits > TBQ4_MAX_SPLITS) return TBQ4_ERR_INVALID_ARG;
  const size_t need = round256((size_t)batch * n_q_heads * n_splits * 130 * sizeof(float));
  if (workspace_bytes < need) return TBQ4_ERR_WORKSPACE;
  if (!aligned16(workspace) || !aligned16(out)) return TBQ4_ERR_ALIGNMENT;
  tbq4::DecodeArgs a;
  memset(&a, 0, sizeof(a));
  a.ws = (float *)workspace;
  a.out = out;
  a.n_q_heads = n_q_heads;
  a.n_splits = n_splits;
  a.rotate_out = 1;
  sign_words(sign_seed, a.sign);
  return from_hip(tbq4::launch_decode_merge(a, batch, (int)out_dtype, (hipStream_t)hip_stream));
}

static_assert(TBQ4_FMT_TBQ4 == tbq4::kFmtTbq4 && TBQ4_FMT_F16 == tbq4::kFmtF16 &&
                  TBQ4_FMT_TBQ3 == tbq4::kFmtTbq3 && TBQ4_FMT_Q8_0 == tbq4::kFmtQ8,
              "format codes of the ABI and the kernels agree");

size_t tbq4_format_row_bytes(int32_t format) {
  switch (format) {
    case TBQ4_FMT_TBQ4: return TBQ4_BLOCK_BYTES;
    case TBQ4_FMT_F16: return 2 * TBQ4_HEAD_DIM;
    case TBQ4_FMT_TBQ3: return tbq4::kBlockBytes3;
    case TBQ4_FMT_Q8_0: return tbq4::kQ8RowBytes;
    default: return 0;
  }
}

// The TBQ4 view of a mixed cache (pointers and shape) for the shared checks,
// plus the checks that depend on the formats.
static tbq4_status mixed_view(const tbq4_mixed_cache *c, tbq4_cache &v) {
  if (!c) return TBQ4_ERR_INVALID_ARG;
  if (tbq4_format_row_bytes(c->k_format) == 0 || tbq4_format_row_bytes(c->v_format) == 0)
    return TBQ4_ERR_UNSUPPORTED;
  v.k = c->k;
  v.v = c->v;
  v.batch = c->batch;
  v.n_kv_heads = c->n_kv_heads;
  v.head_dim = c->head_dim;
  v.capacity = c->capacity;
  v.sign_seed = c->sign_seed;
  tbq4_status s = check_cache(&v);
  if (s != TBQ4_OK) return s;
  if ((int64_t)c->capacity * 2 * TBQ4_HEAD_DIM > 0x7FFFFFF0ll) return TBQ4_ERR_UNSUPPORTED;
  return TBQ4_OK;
}

tbq4_status tbq4_mixed_append(const tbq4_mixed_cache *cache, const void *k_new, const void *v_new,
                              tbq4_dtype src_dtype, int32_t pos, int32_t n_new, void *hip_stream) {
  tbq4_cache view;
  tbq4_status s = mixed_view(cache, view);
  if (s != TBQ4_OK) return s;
  if (!valid_dtype(src_dtype)) return TBQ4_ERR_INVALID_ARG;
  if (n_new < 0 || pos < 0) return TBQ4_ERR_INVALID_ARG;
  if ((int64_t)pos + n_new > cache->capacity) return TBQ4_ERR_CAPACITY;
  if (n_new == 0) return TBQ4_OK;
  if (!k_new || !v_new) return TBQ4_ERR_INVALID_ARG;
  if (!aligned16(k_new) || !aligned16(v_new)) return TBQ4_ERR_ALIGNMENT;
  const void *src[2] = {k_new, v_new};
  uint8_t *dst[2] = {cache->k, cache->v};
  const int32_t fmt[2] = {cache->k_format, cache->v_format};
  uint32_t w[4];
  sign_words(cache->sign_seed, w);
  for (int t = 0; t < 2; ++t) {
    hipError_t e;
    if (fmt[t] == TBQ4_FMT_TBQ4 || fmt[t] == TBQ4_FMT_TBQ3) {
      tbq4::QuantArgs a;
      memset(&a, 0, sizeof(a));
      a.src[0] = src[t];
      a.dst[0] = dst[t];
      a.blocks_per_tensor = (int64_t)cache->batch * n_new * cache->n_kv_heads;
      a.n_new = n_new;
      a.n_kv_heads = cache->n_kv_heads;
      a.capacity = cache->capacity;
      a.pos = pos;
      a.sign_lo = w[0]; a.sign_hi = w[1]; a.sign_lo2 = w[2]; a.sign_hi2 = w[3];
      e = tbq4::launch_quantize(a, (int)src_dtype, 1, (hipStream_t)hip_stream,
                                fmt[t] == TBQ4_FMT_TBQ3 ? tbq4::kFmtTbq3 : tbq4::kFmtTbq4);
    } else if (fmt[t] == TBQ4_FMT_F16) {
      tbq4::StoreF16Args a;
      a.src = src[t];
      a.dst = (_Float16 *)dst[t];
      a.n_groups = (int64_t)cache->batch * n_new * cache->n_kv_heads * (TBQ4_HEAD_DIM / 8);
      a.n_new = n_new;
      a.n_kv_heads = cache->n_kv_heads;
      a.capacity = cache->capacity;
      a.pos = pos;
      e = tbq4::launch_store_f16(a, (int)src_dtype, (hipStream_t)hip_stream);
    } else {
      tbq4::StoreQ8Args a;
      a.src = src[t];
      a.dst = dst[t];
      a.n_blocks = (int64_t)cache->batch * n_new * cache->n_kv_heads * (TBQ4_HEAD_DIM / 32);
      a.n_new = n_new;
      a.n_kv_heads = cache->n_kv_heads;
      a.capacity = cache->capacity;
      a.pos = pos;
      e = tbq4::launch_store_q8(a, (int)src_dtype, (hipStream_t)hip_stream);
    }
    s = from_hip(e);
    if (s != TBQ4_OK) return s;
  }
  return TBQ4_OK;
}

tbq4_status tbq4_mixed_attn_decode(const tbq4_mixed_cache *cache, const void *q,
                                   tbq4_dtype q_dtype, int32_t n_q_heads, int32_t n_ctx,
                                   float softmax_scale, void *out, tbq4_dtype out_dtype,
                                   int32_t n_splits, void *workspace, size_t workspace_bytes,
                                   void *hip_stream) {
  tbq4_cache view;
  tbq4_status s = mixed_view(cache, view);
  if (s != TBQ4_OK) return s;
  if (!out) return TBQ4_ERR_INVALID_ARG;
  if (out_dtype != TBQ4_F32 && out_dtype != TBQ4_F16) return TBQ4_ERR_INVALID_ARG;
  tbq4::DecodeArgs a;
  s = prepare_decode(&view, q, q_dtype, n_q_heads, n_ctx, softmax_scale, n_splits, workspace,
                     workspace_bytes, a);
  if (s != TBQ4_OK) return s;
  if (!aligned16(out)) return TBQ4_ERR_ALIGNMENT;
  a.out = out;
  a.k_fmt = cache->k_format;
  a.v_fmt = cache->v_format;
  a.rotate_out = cache->v_format == TBQ4_FMT_TBQ4 || cache->v_format == TBQ4_FMT_TBQ3 ? 1 : 0;
  hipStream_t st = (hipStream_t)hip_stream;
  s = from_hip(tbq4::launch_decode_partial(a, cache->batch, (int)q_dtype, st));
  if (s != TBQ4_OK) return s;
  return from_hip(tbq4::launch_decode_merge(a, cache->batch, (int)out_dtype, st));
}

int32_t verify_auto_splits(int32_t batch, int32_t n_kv_heads, int32_t n_q, int32_t n_kv) {
  // two wavefronts per SIMD (both kernels fit: q' waits in LDS)
  const int64_t waves = 2048;
  (void)n_q;
  const int64_t n_tiles = (n_kv + tbq4::kDecodeTile - 1) / tbq4::kDecodeTile;
  const int64_t rows = (int64_t)batch * n_kv_heads;
  int64_t p = (waves + rows - 1) / rows;
  const int64_t max_by_len = (n_tiles + 3) / 4;
  if (p > max_by_len) p = max_by_len;
  if (p < 1) p = 1;
  if (p > TBQ4_MAX_SPLITS) p = TBQ4_MAX_SPLITS;
  return (int32_t)p;
}

size_t tbq4_verify_workspace_bytes(int32_t batch, int32_t n_kv_heads, int32_t n_q_heads,
                                   int32_t n_past, int32_t n_q, int32_t n_splits) {
  if (batch <= 0 || n_kv_heads <= 0 || n_q_heads <= 0 || n_q < 1 || n_q > 4 || n_past < 0)
    return 0;
  const int32_t p =
      n_splits == 0 ? verify_auto_splits(batch, n_kv_heads, n_q, n_past + n_q) : n_splits;
  if (p < 1 || p > TBQ4_MAX_SPLITS) return 0;
  return round256((size_t)batch * n_q * n_q_heads * p * 130 * sizeof(float));
}

// Verify over a cache view whose K and V tensors are stored in k_fmt / v_fmt
// (TBQ4, fp16, TBQ3 or q8_0); the caller has checked the view.
static tbq4_status verify_formats(const tbq4_cache *cache, int32_t k_fmt, int32_t v_fmt,
                                  const void *q, tbq4_dtype q_dtype, int32_t n_q_heads,
                                  int32_t n_past, int32_t n_q, float softmax_scale, void *out,
                                  tbq4_dtype out_dtype, int32_t n_splits, void *workspace,
                                  size_t workspace_bytes, void *hip_stream) {
  tbq4_status s;
  if (!q || !out) return TBQ4_ERR_INVALID_ARG;
  if (!valid_dtype(q_dtype)) return TBQ4_ERR_INVALID_ARG;   // fp32, fp16 or bf16
  if (out_dtype != TBQ4_F32 && out_dtype != TBQ4_F16) return TBQ4_ERR_INVALID_ARG;
  if (!isfinite(softmax_scale)) return TBQ4_ERR_INVALID_ARG;
  if (n_q_heads <= 0 || n_q_heads % cache->n_kv_heads != 0) return TBQ4_ERR_UNSUPPORTED;
  const int32_t G = n_q_heads / cache->n_kv_heads;
  if (G > 8) return TBQ4_ERR_UNSUPPORTED;
  if (n_q < 1 || n_q > 4) return TBQ4_ERR_UNSUPPORTED;
  if (n_past < 0) return TBQ4_ERR_INVALID_ARG;
  if ((int64_t)n_past + n_q > cache->capacity) return TBQ4_ERR_CAPACITY;
  if (n_splits < 0 || n_splits > TBQ4_MAX_SPLITS) return TBQ4_ERR_INVALID_ARG;
  if (cache->batch > 65535 || cache->n_kv_heads > 65535 || (int64_t)cache->batch * n_q > 65535)
    return TBQ4_ERR_UNSUPPORTED;
  const int32_t P = n_splits == 0 ? verify_auto_splits(cache->batch, cache->n_kv_heads, n_q,
                                                       n_past + n_q)
                                  : n_splits;
  const size_t need = tbq4_verify_workspace_bytes(cache->batch, cache->n_kv_heads, n_q_heads,
                                                  n_past, n_q, P);
  if (!workspace || workspace_bytes < need) return TBQ4_ERR_WORKSPACE;
  if (!aligned16(workspace) || !aligned16(q) || !aligned16(out)) return TBQ4_ERR_ALIGNMENT;
  tbq4::VerifyArgs a;
  memset(&a, 0, sizeof(a));
  a.k = cache->k;
  a.v = cache->v;
  a.q = q;
  a.ws = (float *)workspace;
  a.n_kv_heads = cache->n_kv_heads;
  a.n_q_heads = n_q_heads;
  a.group = G;
  a.capacity = cache->capacity;
  a.n_past = n_past;
  a.n_q = n_q;
  a.n_splits = P;
  a.qscale = softmax_scale * 1.4426950408889634f;
  sign_words(cache->sign_seed, a.sign);
  a.k_fmt = k_fmt;
  a.v_fmt = v_fmt;
  hipStream_t st = (hipStream_t)hip_stream;
  s = from_hip(tbq4::launch_verify_partial(a, cache->batch, (int)q_dtype, st));
  if (s != TBQ4_OK) return s;
  // merge: row (b, query) of the decode layout, output [B][n_q][Hq][128]
  tbq4::DecodeArgs m;
  memset(&m, 0, sizeof(m));
  m.ws = (float *)workspace;
  m.out = out;
  m.n_q_heads = n_q_heads;
  m.n_splits = P;
  m.rotate_out = v_fmt == TBQ4_FMT_TBQ4 || v_fmt == TBQ4_FMT_TBQ3 ? 1 : 0;
  memcpy(m.sign, a.sign, sizeof(a.sign));
  return from_hip(tbq4::launch_decode_merge(m, cache->batch * n_q, (int)out_dtype, st));
}

tbq4_status tbq4_attn_verify(const tbq4_cache *cache, const void *q, tbq4_dtype q_dtype,
                             int32_t n_q_heads, int32_t n_past, int32_t n_q, float softmax_scale,
                             void *out, tbq4_dtype out_dtype, int32_t n_splits, void *workspace,
                             size_t workspace_bytes, void *hip_stream) {
  tbq4_status s = check_cache(cache);
  if (s != TBQ4_OK) return s;
  return verify_formats(cache, TBQ4_FMT_TBQ4, TBQ4_FMT_TBQ4, q, q_dtype, n_q_heads, n_past, n_q,
                        softmax_scale, out, out_dtype, n_splits, workspace, workspace_bytes,
                        hip_stream);
}

tbq4_status tbq4_mixed_attn_verify(const tbq4_mixed_cache *cache, const void *q,
                                   tbq4_dtype q_dtype, int32_t n_q_heads, int32_t n_past,
                                   int32_t n_q, float softmax_scale, void *out,
                                   tbq4_dtype out_dtype, int32_t n_splits, void *workspace,
                                   size_t workspace_bytes, void *hip_stream) {
  tbq4_cache view;
  tbq4_status s = mixed_view(cache, view);
  if (s != TBQ4_OK) return s;
  return verify_formats(&view, cache->k_format, cache->v_format, q, q_dtype, n_q_heads, n_past,
                        n_q, softmax_scale, out, out_dtype, n_splits, workspace, workspace_bytes,
                        hip_stream);
}

tbq4_status tbq4_quantize_append_at(const tbq4_cache *cache, const void *k_new, const void *v_new,
                                    tbq4_dtype src_dtype, const int32_t *positions, int32_t n_new,
                                    void *hip_stream) {
  tbq4_status s = check_cache(cache);
  if (s != TBQ4_OK) return s;
  if (!valid_dtype(src_dtype)) return TBQ4_ERR_INVALID_ARG;
  if (n_new < 0 || n_new > cache->capacity) return TBQ4_ERR_CAPACITY;
  if (n_new == 0) return TBQ4_OK;
  if (!k_new || !v_new || !positions) return TBQ4_ERR_INVALID_ARG;
  if (!aligned16(k_new) || !aligned16(v_new)) return TBQ4_ERR_ALIGNMENT;
  tbq4::QuantArgs a;
  memset(&a, 0, sizeof(a));
  a.src[0] = k_new;
  a.src[1] = v_new;
  a.dst[0] = cache->k;
  a.dst[1] = cache->v;
  a.blocks_per_tensor = (int64_t)cache->batch * n_new * cache->n_kv_heads;
  a.n_new = n_new;
  a.n_kv_heads = cache->n_kv_heads;
  a.capacity = cache->capacity;
  a.pos_dev = positions;
  uint32_t w[4];
  sign_words(cache->sign_seed, w);
  a.sign_lo = w[0]; a.sign_hi = w[1]; a.sign_lo2 = w[2]; a.sign_hi2 = w[3];
  return from_hip(tbq4::launch_quantize(a, (int)src_dtype, 2, (hipStream_t)hip_stream));
}

tbq4_status tbq4_attn_decode_varlen(const tbq4_cache *cache, const void *q, tbq4_dtype q_dtype,
                                    int32_t n_q_heads, const int32_t *ctx_lens, int32_t max_ctx,
                                    float softmax_scale, void *out, tbq4_dtype out_dtype,
                                    int32_t n_splits, void *workspace, size_t workspace_bytes,
                                    void *hip_stream) {
  if (!out || !ctx_lens) return TBQ4_ERR_INVALID_ARG;
  if (out_dtype != TBQ4_F32 && out_dtype != TBQ4_F16) return TBQ4_ERR_INVALID_ARG;
  tbq4::DecodeArgs a;
  tbq4_status s = prepare_decode(cache, q, q_dtype, n_q_heads, max_ctx, softmax_scale, n_splits,
                                 workspace, workspace_bytes, a);
  if (s != TBQ4_OK) return s;
  if (!aligned16(out)) return TBQ4_ERR_ALIGNMENT;
  a.out = out;
  a.ctx_lens = ctx_lens;
  hipStream_t st = (hipStream_t)hip_stream;
  s = from_hip(tbq4::launch_decode_partial(a, cache->batch, (int)q_dtype, st));
  if (s != TBQ4_OK) return s;
  return from_hip(tbq4::launch_decode_merge(a, cache->batch, (int)out_dtype, st));
}

size_t tbq4_decode_step_workspace_bytes(int32_t batch, int32_t n_kv_heads, int32_t n_q_heads,
                                        int32_t n_ctx, int32_t n_splits) {
  if (batch <= 0 || n_kv_heads <= 0 || n_q_heads <= 0 || n_ctx <= 0) return 0;
  if (n_splits < 0 || n_splits > TBQ4_MAX_SPLITS) return 0;
  const int32_t p = n_splits == 0 ? auto_splits(batch, n_kv_heads, n_ctx) : n_splits;
  return round256((size_t)batch * n_q_heads * (p + 1) * 130 * sizeof(float));
}

static tbq4_status decode_step(const tbq4_cache *cache, const void *k_new, const void *v_new,
                               tbq4_dtype src_dtype, int32_t pos, const int32_t *positions,
                               const void *q, tbq4_dtype q_dtype, int32_t n_q_heads,
                               float softmax_scale, void *out, tbq4_dtype out_dtype,
                               int32_t n_splits, void *workspace, size_t workspace_bytes,
                               void *hip_stream, void *start_event, void *stop_event) {
  if (!out || !k_new || !v_new) return TBQ4_ERR_INVALID_ARG;
  if (out_dtype != TBQ4_F32 && out_dtype != TBQ4_F16) return TBQ4_ERR_INVALID_ARG;
  if (!valid_dtype(src_dtype)) return TBQ4_ERR_INVALID_ARG;
  if (pos < 0) return TBQ4_ERR_CAPACITY;
  if (pos == INT32_MAX) return TBQ4_ERR_CAPACITY;
  // the checks of a decode over pos + 1 slots (capacity, heads, split count)
  // with a stand-in workspace; the step's own size is checked below
  tbq4::DecodeArgs a;
  tbq4_status s = prepare_decode(cache, q, q_dtype, n_q_heads, pos + 1, softmax_scale, n_splits,
                                 reinterpret_cast<void *>((uintptr_t)256), (size_t)-1, a);
  if (s != TBQ4_OK) return s;
  if (a.n_splits + 1 > TBQ4_MAX_SPLITS) return TBQ4_ERR_INVALID_ARG;
  const size_t need = tbq4_decode_step_workspace_bytes(cache->batch, cache->n_kv_heads, n_q_heads,
                                                       pos + 1, a.n_splits);
  if (!workspace || workspace_bytes < need) return TBQ4_ERR_WORKSPACE;
  if (!aligned16(workspace) || !aligned16(out)) return TBQ4_ERR_ALIGNMENT;
  if (!aligned16(k_new) || !aligned16(v_new)) return TBQ4_ERR_ALIGNMENT;
  a.ws = (float *)workspace;
  a.out = out;
  a.n_ctx = pos;                // the streaming splits stop before the new token
  a.ctx_lens = positions;       // (device mode: the token's slot per sequence)
  a.n_splits += 1;              // the new token's partial state comes last
  if ((int64_t)(a.n_splits + 1) * cache->n_kv_heads * cache->batch > 0x7FFFFFFF)
    return TBQ4_ERR_UNSUPPORTED;  // one 1-D grid holds every wavefront
  a.step = 1;
  a.new_dtype = (int32_t)src_dtype;
  a.k_new = k_new;
  a.v_new = v_new;
  hipStream_t st = (hipStream_t)hip_stream;
  s = from_hip(tbq4::launch_decode_partial(a, cache->batch, (int)q_dtype, st,
                                           (hipEvent_t)start_event, (hipEvent_t)stop_event));
  if (s != TBQ4_OK) return s;
  return from_hip(tbq4::launch_decode_merge(a, cache->batch, (int)out_dtype, st));
}

tbq4_status tbq4_decode_step(const tbq4_cache *cache, const void *k_new, const void *v_new,
                             tbq4_dtype src_dtype, int32_t pos, const int32_t *positions,
                             const void *q, tbq4_dtype q_dtype, int32_t n_q_heads,
                             float softmax_scale, void *out, tbq4_dtype out_dtype,
                             int32_t n_splits, void *workspace, size_t workspace_bytes,
                             void *hip_stream) {
  return decode_step(cache, k_new, v_new, src_dtype, pos, positions, q, q_dtype, n_q_heads,
                     softmax_scale, out, out_dtype, n_splits, workspace, workspace_bytes,
                     hip_stream, nullptr, nullptr);
}

tbq4_status tbq4_decode_step_timed(const tbq4_cache *cache, const void *k_new, const void *v_new,
                                   tbq4_dtype src_dtype, int32_t pos, const int32_t *positions,
                                   const void *q, tbq4_dtype q_dtype, int32_t n_q_heads,
                                   float softmax_scale, void *out, tbq4_dtype out_dtype,
                                   int32_t n_splits, void *workspace, size_t workspace_bytes,
                                   void *hip_stream, void *start_event, void *stop_event) {
  return decode_step(cache, k_new, v_new, src_dtype, pos, positions, q, q_dtype, n_q_heads,
                     softmax_scale, out, out_dtype, n_splits, workspace, workspace_bytes,
                     hip_stream, start_event, stop_event);
}

// Prefill on K / V tensors in the given formats (TBQ4, fp16, TBQ3 or q8_0);
// the cache view has been checked.
static tbq4_status prefill_formats(const tbq4_cache *cache, int32_t k_fmt, int32_t v_fmt,
                                   const void *q, tbq4_dtype q_dtype, int32_t n_q_heads,
                                   int32_t n_past, int32_t n_q, float softmax_scale, void *out,
                                   tbq4_dtype out_dtype, void *hip_stream) {
  if (!q || !out) return TBQ4_ERR_INVALID_ARG;
  if (!valid_dtype(q_dtype)) return TBQ4_ERR_INVALID_ARG;   // fp32, fp16 or bf16
  if (out_dtype != TBQ4_F32 && out_dtype != TBQ4_F16) return TBQ4_ERR_INVALID_ARG;
  if (!isfinite(softmax_scale)) return TBQ4_ERR_INVALID_ARG;
  if (n_q_heads <= 0 || n_q_heads % cache->n_kv_heads != 0) return TBQ4_ERR_UNSUPPORTED;
  const int32_t G = n_q_heads / cache->n_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16 && G != 32) return TBQ4_ERR_UNSUPPORTED;
  if (n_past < 0 || n_q < 1) return TBQ4_ERR_CAPACITY;
  if ((int64_t)n_past + n_q > cache->capacity) return TBQ4_ERR_CAPACITY;
  if (!aligned16(q) || !aligned16(out)) return TBQ4_ERR_ALIGNMENT;
  tbq4::PrefillArgs a;
  memset(&a, 0, sizeof(a));
  a.k = cache->k;
  a.v = cache->v;
  a.q = q;
  a.out = out;
  a.n_kv_heads = cache->n_kv_heads;
  a.n_q_heads = n_q_heads;
  a.group = G;
  a.capacity = cache->capacity;
  a.n_past = n_past;
  a.n_q = n_q;
  a.qscale = softmax_scale * 1.4426950408889634f;
  sign_words(cache->sign_seed, a.sign);
  a.k_fmt = k_fmt;
  a.v_fmt = v_fmt;
  return from_hip(tbq4::launch_prefill(a, cache->batch, (int)q_dtype, (int)out_dtype,
                                       (hipStream_t)hip_stream));
}

tbq4_status tbq4_attn_prefill_chunk(const tbq4_cache *cache, const void *q, tbq4_dtype q_dtype,
                                    int32_t n_q_heads, int32_t n_past, int32_t n_q,
                                    float softmax_scale, void *out, tbq4_dtype out_dtype,
                                    void *hip_stream) {
  tbq4_status s = check_cache(cache);
  if (s != TBQ4_OK) return s;
  return prefill_formats(cache, TBQ4_FMT_TBQ4, TBQ4_FMT_TBQ4, q, q_dtype, n_q_heads, n_past, n_q,
                         softmax_scale, out, out_dtype, hip_stream);
}

tbq4_status tbq4_mixed_attn_prefill_chunk(const tbq4_mixed_cache *cache, const void *q,
                                          tbq4_dtype q_dtype, int32_t n_q_heads, int32_t n_past,
                                          int32_t n_q, float softmax_scale, void *out,
                                          tbq4_dtype out_dtype, void *hip_stream) {
  tbq4_cache view;
  tbq4_status s = mixed_view(cache, view);
  if (s != TBQ4_OK) return s;
  return prefill_formats(&view, cache->k_format, cache->v_format, q, q_dtype, n_q_heads, n_past,
                         n_q, softmax_scale, out, out_dtype, hip_stream);
}

const char *tbq4_status_str(tbq4_status s) {
  switch (s) {
    case TBQ4_OK: return "ok";
    case TBQ4_ERR_INVALID_ARG: return "invalid argument";
    case TBQ4_ERR_UNSUPPORTED: return "unsupported shape";
    case TBQ4_ERR_CAPACITY: return "token range exceeds cache capacity";
    case TBQ4_ERR_ALIGNMENT: return "pointer or capacity not aligned";
    case TBQ4_ERR_WORKSPACE: return "workspace missing or too small";
    case TBQ4_ERR_HIP: return "HIP launch error";
  }
  return "unknown status";
}

const char *tbq4_version(void) { return "0.1.0"; }

}  // extern "C"
