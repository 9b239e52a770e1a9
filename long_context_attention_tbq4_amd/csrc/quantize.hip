// TBQ4 / TBQ3 quantise-and-pack kernel (the write side of the cache): one
// wavefront per block, the arithmetic of tbq4_quant.h (page "Kontekst 262K
// na jednej RTX 4090: co dodałem do llama.cpp-turboq", section "Od czego
// zacząłem": 128 values -> a 2-byte scale and 64 bytes of 4-bit indices in
// the rotated Hadamard domain).  Also the plain fp16 and q8_0 row stores of
// the mixed-format caches.
#include "tbq4_device.h"
#include "tbq4_launch.h"
#include "tbq4_quant.h"

namespace tbq4 {

#pragma clang fp contract(off)

template <typename T, int FMT>
__global__ __launch_bounds__(256) void quantize_kernel(QuantArgs a) {
  constexpr int64_t kBB = FMT == kFmtTbq3 ? kBlockBytes3 : kBlockBytes;   // bytes per block
  const int lane = threadIdx.x & 63;
  const int64_t gblock = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tensor = gblock >= a.blocks_per_tensor ? 1 : 0;
  const int64_t i = gblock - (int64_t)tensor * a.blocks_per_tensor;
  // the grid is rounded up to whole 4-wavefront workgroups: wavefronts past
  // the last tensor of this launch (one or two tensors) have no block
  if (tensor >= a.n_tensors) return;
  if (i >= a.blocks_per_tensor) return;

  const T *src;
  uint8_t *dst;
  if (a.flat) {
    src = (const T *)a.src[0] + i * kHeadDim;
    dst = a.dst[0] + i * kBB;
  } else {
    // source [batch][n_new][n_kv_heads][128]; cache [batch][n_kv_heads][capacity][66]
    int64_t h, t, b;
    if (a.blocks_per_tensor <= 0x7FFFFFFF) {   // 32-bit index arithmetic
      const uint32_t i32 = (uint32_t)i, nh = (uint32_t)a.n_kv_heads, nn = (uint32_t)a.n_new;
      const uint32_t q = i32 / nh;
      h = i32 - q * nh;
      t = q % nn;
      b = q / nn;
    } else {
      h = i % a.n_kv_heads;
      t = (i / a.n_kv_heads) % a.n_new;
      b = i / ((int64_t)a.n_kv_heads * a.n_new);
    }
    // first slot of this sequence: a host value, or per sequence from device
    // memory (slots outside [0, capacity) are skipped; the whole wavefront
    // leaves together)
    const int64_t slot = (a.pos_dev ? (int64_t)a.pos_dev[b] : (int64_t)a.pos) + t;
    if (slot < 0 || slot >= a.capacity) return;
    src = (const T *)a.src[tensor] + i * kHeadDim;
    dst = a.dst[tensor] + ((b * a.n_kv_heads + h) * a.capacity + slot) * kBB;
  }

  const LaneCodes c = quantize_lanes<T, FMT>(src, lane < 32 ? a.sign_lo : a.sign_hi,
                                             lane < 32 ? a.sign_lo2 : a.sign_hi2, lane);
  store_lanes<FMT>(dst, c, lane);
}


// fp16 cache rows (the mixed-format caches): x -> binary16, round to nearest
// even (overflow to infinity), one thread per 8 consecutive values.  Source
// [batch][n_new][n_kv_heads][128]; destination [batch][n_kv_heads][capacity][128]
// fp16 at slots pos .. pos + n_new - 1.
template <typename T>
__global__ __launch_bounds__(256) void store_f16_kernel(StoreF16Args a) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;   // group of 8 values
  if (i >= a.n_groups) return;
  const int64_t vec = i >> 4;                                   // head vector
  const int dim0 = (int)(i & 15) * 8;
  const int64_t h = vec % a.n_kv_heads;
  const int64_t t = (vec / a.n_kv_heads) % a.n_new;
  const int64_t b = vec / ((int64_t)a.n_kv_heads * a.n_new);
  const T *src = (const T *)a.src + vec * kHeadDim + dim0;
  _Float16 *dst = a.dst + ((b * a.n_kv_heads + h) * a.capacity + a.pos + t) * kHeadDim + dim0;
  half8 v;
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = (_Float16)(float)load_exact<T>(src + e);
  *(half8 *)dst = v;
}

hipError_t launch_store_f16(const StoreF16Args &a, int dtype, hipStream_t stream) {
  const int64_t grid = (a.n_groups + 255) / 256;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  switch (dtype) {
    case 0: hipLaunchKernelGGL(store_f16_kernel<float>, dim3((unsigned)grid), dim3(256), 0, stream, a); break;
    case 1: hipLaunchKernelGGL(store_f16_kernel<_Float16>, dim3((unsigned)grid), dim3(256), 0, stream, a); break;
    default: hipLaunchKernelGGL(store_f16_kernel<uint16_t>, dim3((unsigned)grid), dim3(256), 0, stream, a); break;
  }
  return hipGetLastError();
}

// q8_0 rows: one thread per value, the 32 lanes of a half-wavefront one
// 32-value block.  d32 = amax / 127 and x / d32 are IEEE fp32 divisions
// (correctly rounded), the code is x / d32 rounded to the nearest integer
// with halves away from zero (roundf), the stored scale is the binary16
// nearest d32.  Source [batch][n_new][n_kv_heads][128]; destination
// [batch][n_kv_heads][capacity][136] at slots pos .. pos + n_new - 1.
template <typename T>
__global__ __launch_bounds__(256) void store_q8_kernel(StoreQ8Args a) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;   // value index
  const int64_t blk = i >> 5;                                   // same for 32 lanes
  const int e = (int)(i & 31);
  const bool live = blk < a.n_blocks;
  const float x = live ? (float)load_exact<T>((const T *)a.src + i) : 0.0f;
  float amax = fabsf(x);
#pragma unroll
  for (int o = 1; o < 32; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
  if (!live) return;
  const float d32 = amax / 127.0f;
  const int q = d32 > 0.0f ? (int)roundf(x / d32) : 0;
  const int64_t vec = blk >> 2;                                 // head vector
  const int kb = (int)(blk & 3);
  const int64_t h = vec % a.n_kv_heads;
  const int64_t t = (vec / a.n_kv_heads) % a.n_new;
  const int64_t b = vec / ((int64_t)a.n_kv_heads * a.n_new);
  uint8_t *dst = a.dst + ((b * a.n_kv_heads + h) * a.capacity + a.pos + t) * kQ8RowBytes + 34 * kb;
  dst[2 + e] = (uint8_t)(int8_t)q;
  if (e == 0) *(uint16_t *)dst = __builtin_bit_cast(uint16_t, (_Float16)d32);
}

hipError_t launch_store_q8(const StoreQ8Args &a, int dtype, hipStream_t stream) {
  const int64_t grid = (a.n_blocks * 32 + 255) / 256;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  switch (dtype) {
    case 0: hipLaunchKernelGGL(store_q8_kernel<float>, dim3((unsigned)grid), dim3(256), 0, stream, a); break;
    case 1: hipLaunchKernelGGL(store_q8_kernel<_Float16>, dim3((unsigned)grid), dim3(256), 0, stream, a); break;
    default: hipLaunchKernelGGL(store_q8_kernel<uint16_t>, dim3((unsigned)grid), dim3(256), 0, stream, a); break;
  }
  return hipGetLastError();
}

template <int FMT>
static void launch_quantize_fmt(const QuantArgs &a, int dtype, unsigned grid, hipStream_t stream) {
  switch (dtype) {
    case 0: hipLaunchKernelGGL((quantize_kernel<float, FMT>), dim3(grid), dim3(256), 0, stream, a); break;
    case 1: hipLaunchKernelGGL((quantize_kernel<_Float16, FMT>), dim3(grid), dim3(256), 0, stream, a); break;
    default: hipLaunchKernelGGL((quantize_kernel<uint16_t, FMT>), dim3(grid), dim3(256), 0, stream, a); break;
  }
}

hipError_t launch_quantize(const QuantArgs &args, int dtype, int tensors, hipStream_t stream,
                           int format) {
  if (tensors < 1 || tensors > 2 || (args.flat && tensors != 1)) return hipErrorInvalidValue;
  if (format != kFmtTbq4 && format != kFmtTbq3) return hipErrorInvalidValue;
  QuantArgs a = args;
  a.n_tensors = tensors;
  const int64_t blocks = a.blocks_per_tensor * tensors;
  const int64_t grid = (blocks + 3) / 4;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (format == kFmtTbq3) launch_quantize_fmt<kFmtTbq3>(a, dtype, (unsigned)grid, stream);
  else launch_quantize_fmt<kFmtTbq4>(a, dtype, (unsigned)grid, stream);
  return hipGetLastError();
}

}  // namespace tbq4
