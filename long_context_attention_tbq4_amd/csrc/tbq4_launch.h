// Internal launch interface between the C-ABI layer and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tbq4 {

struct QuantArgs {
  const void *src[2];          // K and V sources (V unused in flat mode)
  uint8_t *dst[2];             // K and V caches (or the flat output)
  int64_t blocks_per_tensor;   // blocks per source tensor
  int32_t n_new, n_kv_heads, capacity, pos;
  int32_t flat;                // 1: block i -> src + 128 i, dst + 66 i
  int32_t n_tensors;           // 1 or 2 tensors in this launch (set by launch_quantize)
  const int32_t *pos_dev;      // device [batch] first slot per sequence, or null (use pos)
  uint32_t sign_lo, sign_hi;   // sign bits 0..31, 32..63
  uint32_t sign_lo2, sign_hi2; // sign bits 64..95, 96..127
};

struct StoreF16Args {
  const void *src;             // [batch][n_new][n_kv_heads][128]
  _Float16 *dst;               // [batch][n_kv_heads][capacity][128]
  int64_t n_groups;            // batch * n_new * n_kv_heads * 16
  int32_t n_new, n_kv_heads, capacity, pos;
};

struct StoreQ8Args {
  const void *src;             // [batch][n_new][n_kv_heads][128]
  uint8_t *dst;                // [batch][n_kv_heads][capacity][136]
  int64_t n_blocks;            // batch * n_new * n_kv_heads * 4 (32-value blocks)
  int32_t n_new, n_kv_heads, capacity, pos;
};

struct DecodeArgs {
  const uint8_t *k;
  const uint8_t *v;
  const void *q;         // [B][Hq][128]
  float *ws;             // [B][Hq][P][130]
  void *out;             // [B][Hq][128]
  const int32_t *ctx_lens;  // device [B] per-sequence lengths (clamped to [0, n_ctx]), or null
  int32_t n_kv_heads, n_q_heads, group, capacity;
  int32_t n_ctx;         // context length, or the upper bound of ctx_lens
  int32_t n_splits;
  int32_t k_fmt, v_fmt;  // cache formats (kFmtTbq4, kFmtF16, kFmtTbq3, kFmtQ8)
  int32_t rotate_out;    // merge applies R^T (the V cache holds rotated values)
  float qscale;          // softmax_scale * log2(e)
  uint32_t sign[4];      // sign bits 0..31, 32..63, 64..95, 96..127
  // Decode step (append + attend in one launch; TBQ K and V): the last of
  // the n_splits partial states of each head is the new token's, written by
  // two extra wavefronts per (sequence, KV head) that also store its blocks.
  // The new token sits at slot ctx_lens[b] (device) or n_ctx (host) and the
  // other splits stream the slots before it; a device slot outside
  // [0, n_ctx] gives that sequence no token and no context.
  int32_t step;          // 0: plain decode; 1: decode step
  int32_t new_dtype;     // dtype of k_new / v_new (0 fp32, 1 fp16, 2 bf16)
  const void *k_new;     // [B][H_kv][128]
  const void *v_new;
};

struct VerifyArgs {
  const uint8_t *k;
  const uint8_t *v;
  const void *q;         // [B][n_q][Hq][128]
  float *ws;             // [B * n_q][Hq][P][130] (the decode layout)
  int32_t n_kv_heads, n_q_heads, group, capacity, n_past, n_q, n_splits;
  float qscale;          // softmax_scale * log2(e)
  uint32_t sign[4];
  int32_t k_fmt, v_fmt;  // cache formats (TBQ4, fp16, TBQ3 or q8_0; zero = TBQ4)
};

struct PrefillArgs {
  const uint8_t *k;
  const uint8_t *v;
  const void *q;         // [B][n_q][Hq][128]
  void *out;             // [B][n_q][Hq][128]
  int32_t n_kv_heads, n_q_heads, group, capacity, n_past, n_q;
  float qscale;          // softmax_scale * log2(e)
  uint32_t sign[4];
  int32_t k_fmt, v_fmt;  // cache formats (TBQ4, fp16 or TBQ3; zero = TBQ4)
};

constexpr int kDecodeTile = 32;

// Cache formats of a K or V tensor: TBQ4 blocks (66 B per head vector), fp16
// rows (256 B, not rotated), TBQ3 blocks (50 B), q8_0 rows (four 34-byte
// blocks of a binary16 scale and 32 int8 codes, 136 B, not rotated).
constexpr int kFmtTbq4 = 0, kFmtF16 = 1, kFmtTbq3 = 2, kFmtQ8 = 3;
constexpr int kNumFormats = 4;
constexpr uint32_t kBlockBytes3 = 50;
constexpr uint32_t kQ8RowBytes = 136;

hipError_t launch_quantize(const QuantArgs &a, int dtype, int tensors, hipStream_t stream,
                           int format = kFmtTbq4);
hipError_t launch_store_f16(const StoreF16Args &a, int dtype, hipStream_t stream);
hipError_t launch_store_q8(const StoreQ8Args &a, int dtype, hipStream_t stream);
// With start/stop events the dispatch itself records them (hipExtLaunchKernel).
hipError_t launch_decode_partial(const DecodeArgs &a, int batch, int q_dtype, hipStream_t stream,
                                 hipEvent_t start = nullptr, hipEvent_t stop = nullptr);
hipError_t launch_decode_merge(const DecodeArgs &a, int batch, int out_dtype, hipStream_t stream);
// Size of the static device array that holds the split-K partial states of
// the no-allocation decode entry point, and its device address on the device
// `stream` runs on (looked up once per device; never the array's host-side
// name).
constexpr size_t kDecodeScratchBytes = (size_t)16 << 20;
hipError_t decode_scratch(hipStream_t stream, void **ptr);
hipError_t launch_verify_partial(const VerifyArgs &a, int batch, int q_dtype, hipStream_t stream);
hipError_t launch_prefill(const PrefillArgs &a, int batch, int q_dtype, int out_dtype,
                          hipStream_t stream);

}  // namespace tbq4
