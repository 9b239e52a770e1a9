// TBQ4 quantise-and-pack kernel (the write side of the cache).
//
// Page "Kontekst 262K na jednej RTX 4090: co dodałem do llama.cpp-turboq",
// section "Od czego zacząłem": a block is 128 values stored in 66 bytes, a
// 2-byte scale then 64 bytes of 4-bit indices, in the rotated Hadamard domain.
// The page does not describe how blocks are written; this kernel fixes every
// step as an IEEE fp64 operation in a stated order so that the bytes are a
// pure function of the input (bit-exact against an independent fp64
// implementation of the same steps):
//   v = s * x                           (s = +-1 from SplitMix64(seed))
//   butterflies h = 1,2,...,64:  (v_i, v_{i+h}) <- (v_i + v_{i+h}, v_i - v_{i+h})
//   u = v * fl64(1/sqrt(128))
//   p = u*u; tree p_i += p_{i+h} for h = 64..1; ms = p_0 * 2^-7
//   d = binary16 nearest sqrt(ms) (exact comparison with squared midpoints,
//       ties to even, saturating at 65504)
//   code_i = 8*[u_i < 0] + #{k < 7 : d * tau_k < |u_i|}, tau_k midpoints of
//       adjacent level magnitudes (nearest level, ties toward zero)
//   bytes: d (LE) then code_{2j} | code_{2j+1} << 4
//
// One wavefront quantises one block: lane l holds elements l and l+64.
#include "tbq4_device.h"
#include "tbq4_launch.h"

namespace tbq4 {

#pragma clang fp contract(off)

// fl64(1/sqrt(128)) = 0x1.6a09e667f3bccp-4
__device__ __forceinline__ double inv_sqrt128() { return __longlong_as_double(0x3FB6A09E667F3BCCll); }

// exact value of binary16 pattern h (0 <= h <= 0x7C00)
__device__ __forceinline__ double half_value(int h) {
  const int e = h >> 10, m = h & 0x3FF;
  return e == 0 ? ldexp((double)m, -24) : ldexp((double)(1024 + m), e - 25);
}

// Pattern of the binary16 value nearest sqrt(ms): the largest h in
// [0, 0x7BFF] whose lower midpoint mid(h) = (value(h-1)+value(h))/2 lies
// below sqrt(ms) -- or equals it with h even.  mid(h) has <= 12 significant
// bits, so mid(h)^2 is exact and the test takes no square root.
__device__ __forceinline__ bool below_sqrt(int h, double ms) {   // 1 <= h <= 0x7BFF
  const double m = (half_value(h - 1) + half_value(h)) * 0.5;
  const double m2 = m * m;
  return (m2 < ms) || (m2 == ms && (h & 1) == 0);
}

// The search starts from sqrt(ms) rounded through binary32 to binary16,
// which is never more than one pattern away from the answer (the rounding
// near every midpoint was checked exhaustively), and moves by the exact test
// above, up to two patterns each way; zero, NaN and overflow give the
// patterns the full search gives (0, 0, 0x7BFF).
__device__ __forceinline__ int half_round_sqrt(double ms) {
  if (!(ms > 0.0)) return 0;
  const _Float16 c = (_Float16)(float)sqrt(ms);
  int h = (int)(__builtin_bit_cast(uint16_t, c) & 0x7FFFu);
  if (h > 0x7BFF) h = 0x7BFF;
#pragma unroll
  for (int k = 0; k < 2; ++k)
    if (h > 0 && !below_sqrt(h, ms)) --h;
#pragma unroll
  for (int k = 0; k < 2; ++k)
    if (h < 0x7BFF && below_sqrt(h + 1, ms)) ++h;
  return h;
}

// x of lane (lane ^ H), H in {1, 2, 4, 8, 16, 32}, without a round trip
// through LDS: DPP quad permutations (1, 2), row shifts restricted to banks
// (4: banks 0 and 2 read four lanes up, banks 1 and 3 four lanes down), a
// row rotation (8), and gfx950's swaps of adjacent 16-lane rows and of the
// two 32-lane halves (16, 32), whose two results hold the partner's value
// for odd and even rows (halves) respectively.
template <int H> __device__ __forceinline__ uint32_t lane_xor(uint32_t x, int lane) {
  if constexpr (H == 1) {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0xB1, 0xF, 0xF, false);
  } else if constexpr (H == 2) {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0x4E, 0xF, 0xF, false);
  } else if constexpr (H == 4) {
    const int t = __builtin_amdgcn_update_dpp((int)x, (int)x, 0x104, 0xF, 0x5, false);
    return (uint32_t)__builtin_amdgcn_update_dpp(t, (int)x, 0x114, 0xF, 0xA, false);
  } else if constexpr (H == 8) {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)x, 0x128, 0xF, 0xF, false);
  } else if constexpr (H == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    return (lane & 16) ? r[0] : r[1];
  } else {
    static_assert(H == 32, "lane_xor: H is a power of two below 64");
    const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return (lane & 32) ? r[0] : r[1];
  }
}
template <int H> __device__ __forceinline__ double lane_xor_f64(double v, int lane) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint64_t lo = lane_xor<H>((uint32_t)b, lane), hi = lane_xor<H>((uint32_t)(b >> 32), lane);
  return __builtin_bit_cast(double, lo | (hi << 32));
}

// One butterfly stage across lanes: (v_i, v_{i+H}) <- (v_i + v_{i+H}, v_i - v_{i+H})
// for the element pair held by lanes i and i + H.
template <int H> __device__ __forceinline__ void butterfly_lanes(double &v, int lane) {
  const double p = lane_xor_f64<H>(v, lane);
  v = (lane & H) ? (p - v) : (v + p);
}
// p_i <- p_i + p_{i+H} for lanes i < H (other lanes compute values nobody reads)
template <int H> __device__ __forceinline__ void fold_lanes(double &p, int lane) {
  p = p + lane_xor_f64<H>(p, lane);
}

template <typename T> __device__ __forceinline__ double load_exact(const T *p);
template <> __device__ __forceinline__ double load_exact<float>(const float *p) { return (double)*p; }
template <> __device__ __forceinline__ double load_exact<_Float16>(const _Float16 *p) { return (double)*p; }
template <> __device__ __forceinline__ double load_exact<uint16_t>(const uint16_t *p) {
  // bf16: the upper half of an fp32
  return (double)__uint_as_float(((uint32_t)*p) << 16);
}


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

  // signs of elements lane and lane+64
  const uint32_t w_a = lane < 32 ? a.sign_lo : a.sign_hi;
  const uint32_t w_b = lane < 32 ? a.sign_lo2 : a.sign_hi2;
  const bool neg0 = (w_a >> (lane & 31)) & 1u;
  const bool neg1 = (w_b >> (lane & 31)) & 1u;
  double v0 = load_exact<T>(src + lane);
  double v1 = load_exact<T>(src + lane + 64);
  if (neg0) v0 = -v0;
  if (neg1) v1 = -v1;

  // butterflies h = 1..32 across lanes, then h = 64 inside the lane
  butterfly_lanes<1>(v0, lane);  butterfly_lanes<1>(v1, lane);
  butterfly_lanes<2>(v0, lane);  butterfly_lanes<2>(v1, lane);
  butterfly_lanes<4>(v0, lane);  butterfly_lanes<4>(v1, lane);
  butterfly_lanes<8>(v0, lane);  butterfly_lanes<8>(v1, lane);
  butterfly_lanes<16>(v0, lane); butterfly_lanes<16>(v1, lane);
  butterfly_lanes<32>(v0, lane); butterfly_lanes<32>(v1, lane);
  {
    const double a0 = v0, b0 = v1;
    v0 = a0 + b0;
    v1 = a0 - b0;
  }
  const double R = inv_sqrt128();
  const double u0 = v0 * R;
  const double u1 = v1 * R;

  // mean square: p_l = u_l^2 + u_{l+64}^2, then p_l += p_{l+h}, h = 32..1
  const double q0 = u0 * u0;
  const double q1 = u1 * u1;
  double p = q0 + q1;
  fold_lanes<32>(p, lane);
  fold_lanes<16>(p, lane);
  fold_lanes<8>(p, lane);
  fold_lanes<4>(p, lane);
  fold_lanes<2>(p, lane);
  fold_lanes<1>(p, lane);
  const uint64_t sb = __builtin_bit_cast(uint64_t, p);
  const double S = __builtin_bit_cast(
      double, (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)sb) |
                  ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(sb >> 32)) << 32));
  const double ms = S * 0x1p-7;
  const int dbits = half_round_sqrt(ms);
  const double d = half_value(dbits);

  const double a0 = fabs(u0), a1 = fabs(u1);
  if constexpr (FMT == kFmtTbq3) {
    // TBQ3: bit 2 = sign, bits 0-1 = number of scaled midpoints of the
    // magnitudes 0.25 0.75 1.375 2.25 below |u|; code i at bits 3i .. 3i+2
    // of the little-endian integer in bytes 2..49
    const double tau3[3] = {0.5, 1.0625, 1.8125};
    int c0 = u0 < 0.0 ? 4 : 0, c1 = u1 < 0.0 ? 4 : 0;
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      const double dt = d * tau3[k];
      c0 += dt < a0 ? 1 : 0;
      c1 += dt < a1 ? 1 : 0;
    }
    // lane w < 12 assembles bits 32w .. 32w+31: the codes i with
    // 3i + 3 > 32w and 3i < 32w + 32 (code i lives in lane i & 63)
    const int both = c0 | (c1 << 8);
    const int w = lane < 12 ? lane : 0;
    const int i_first = (32 * w) / 3;
    uint32_t word = 0;
#pragma unroll
    for (int k = 0; k < 12; ++k) {
      const int i = i_first + k;
      const int src = __shfl(both, i & 63, 64);
      const uint32_t c = (uint32_t)((i >= 64 ? src >> 8 : src) & 7);
      const int off = 3 * i - 32 * w;
      if (i < 128 && off < 32) word |= off >= 0 ? (c << off) : (c >> -off);
    }
    // 24 half-words at byte 2 + 2j (block starts are 2-byte aligned)
    const uint32_t wj = (uint32_t)__shfl((int)word, (lane >> 1) & 15, 64);
    if (lane < 24) *(uint16_t *)(dst + 2 + 2 * lane) = (uint16_t)(wj >> (16 * (lane & 1)));
    if (lane == 0) *(uint16_t *)dst = (uint16_t)dbits;
    return;
  }

  // sign-magnitude code: bit 3 = sign of u, bits 0-2 = number of scaled
  // magnitude midpoints strictly below |u| (d * tau_k is exact)
  const double tau[7] = {0.25, 0.5, 0.78125, 1.09375, 1.4375, 1.8125, 2.375};
  int i0 = u0 < 0.0 ? 8 : 0, i1 = u1 < 0.0 ? 8 : 0;
#pragma unroll
  for (int k = 0; k < 7; ++k) {
    const double dt = d * tau[k];
    i0 += dt < a0 ? 1 : 0;
    i1 += dt < a1 ? 1 : 0;
  }

  // byte m = code[2m] | code[2m+1] << 4.  Elements 2m and 2m+1 sit in the
  // adjacent lanes 2m and 2m+1 (m < 32, first element) or 2m-64 and 2m-63
  // (m >= 32, second element): an even lane e forms bytes e/2 and 32 + e/2
  // with its odd neighbour's codes, and a lane e = 4k joins them with lane
  // e + 2's into two 16-bit words, bytes 2k, 2k+1 and 32+2k, 33+2k.
  const uint32_t both = (uint32_t)(i0 | (i1 << 16));                 // codes < 16
  const uint32_t pair = both | (lane_xor<1>(both, lane) << 4);      // even lanes
  const uint32_t quad = pair | (lane_xor<2>(pair, lane) << 8);      // lanes 4k
  if ((lane & 3) == 0) {
    *(uint16_t *)(dst + 2 + (lane >> 1)) = (uint16_t)(quad & 0xFFFFu);
    *(uint16_t *)(dst + 34 + (lane >> 1)) = (uint16_t)(quad >> 16);
  }
  if (lane == 0) *(uint16_t *)dst = (uint16_t)dbits;
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
