// The block quantiser's arithmetic, shared by the append kernel and the
// decode step's new-token wavefront (one wavefront per block: lane l holds
// elements l and l + 64).
//
// Page "Kontekst 262K na jednej RTX 4090: co dodałem do llama.cpp-turboq",
// section "Od czego zacząłem": a block is 128 values stored in 66 bytes, a
// 2-byte scale then 64 bytes of 4-bit indices, in the rotated Hadamard domain.
// The page does not describe how blocks are written; every step here is an
// IEEE fp64 operation in a stated order, so the bytes are a pure function of
// the input:
//   v = s * x                           (s = +-1 from SplitMix64(seed))
//   butterflies h = 1,2,...,64:  (v_i, v_{i+h}) <- (v_i + v_{i+h}, v_i - v_{i+h})
//   u = v * fl64(1/sqrt(128))
//   p = u*u; tree p_i += p_{i+h} for h = 64..1; ms = p_0 * 2^-7
//   d = binary16 nearest sqrt(ms) (exact comparison with squared midpoints,
//       ties to even, saturating at 65504)
//   code_i = 8*[u_i < 0] + #{k < 7 : d * tau_k < |u_i|}, tau_k midpoints of
//       adjacent level magnitudes (nearest level, ties toward zero)
//   bytes: d (LE) then code_{2j} | code_{2j+1} << 4
// (TBQ3: the same rotation and scale, 4 magnitudes, 3-bit codes.)
// Every function that does fp64 arithmetic turns contraction off in its own
// body, so the operations stay unfused wherever the code is inlined.
#pragma once
#include "tbq4_device.h"
#include "tbq4_launch.h"

namespace tbq4 {

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
#pragma clang fp contract(off)
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
#pragma clang fp contract(off)
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

// Rotated elements and codes of one block, as lane `lane` holds them:
// element lane (c0, u0) and lane + 64 (c1, u1); dbits = the scale's pattern.
struct LaneCodes {
  int c0, c1;
  int dbits;
};

// Quantise the block at `src` (128 values of type T: fp32, fp16 or bf16 as
// uint16_t); w_a / w_b hold the sign bits of elements lane and lane + 64
// (bits 0-31 / 32-63 of the sign vector for lanes below 32, else the word
// after; bits 64-127 likewise for w_b).
// quantize_values: the same from the two values already loaded (x0 =
// element lane, x1 = element lane + 64, exact in fp64).
template <int FMT>
__device__ __forceinline__ LaneCodes quantize_values(double v0, double v1, uint32_t w_a,
                                                     uint32_t w_b, int lane) {
#pragma clang fp contract(off)
  const bool neg0 = (w_a >> (lane & 31)) & 1u;
  const bool neg1 = (w_b >> (lane & 31)) & 1u;
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
    // magnitudes 0.25 0.75 1.375 2.25 below |u|
    const double tau3[3] = {0.5, 1.0625, 1.8125};
    int c0 = u0 < 0.0 ? 4 : 0, c1 = u1 < 0.0 ? 4 : 0;
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      const double dt = d * tau3[k];
      c0 += dt < a0 ? 1 : 0;
      c1 += dt < a1 ? 1 : 0;
    }
    return {c0, c1, dbits};
  } else {
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
    return {i0, i1, dbits};
  }
}

template <typename T, int FMT>
__device__ __forceinline__ LaneCodes quantize_lanes(const T *src, uint32_t w_a, uint32_t w_b,
                                                   int lane) {
  return quantize_values<FMT>(load_exact<T>(src + lane), load_exact<T>(src + lane + 64), w_a, w_b,
                              lane);
}

// Write the block's bytes at dst (a block start: 2-byte aligned).
template <int FMT>
__device__ __forceinline__ void store_lanes(uint8_t *dst, const LaneCodes &c, int lane) {
  if constexpr (FMT == kFmtTbq3) {
    // code i at bits 3i .. 3i+2 of the little-endian integer in bytes 2..49;
    // lane w < 12 assembles bits 32w .. 32w+31: the codes i with
    // 3i + 3 > 32w and 3i < 32w + 32 (code i lives in lane i & 63)
    const int both = c.c0 | (c.c1 << 8);
    const int w = lane < 12 ? lane : 0;
    const int i_first = (32 * w) / 3;
    uint32_t word = 0;
#pragma unroll
    for (int k = 0; k < 12; ++k) {
      const int i = i_first + k;
      const int src = __shfl(both, i & 63, 64);
      const uint32_t cc = (uint32_t)((i >= 64 ? src >> 8 : src) & 7);
      const int off = 3 * i - 32 * w;
      if (i < 128 && off < 32) word |= off >= 0 ? (cc << off) : (cc >> -off);
    }
    // 24 half-words at byte 2 + 2j (block starts are 2-byte aligned)
    const uint32_t wj = (uint32_t)__shfl((int)word, (lane >> 1) & 15, 64);
    if (lane < 24) *(uint16_t *)(dst + 2 + 2 * lane) = (uint16_t)(wj >> (16 * (lane & 1)));
    if (lane == 0) *(uint16_t *)dst = (uint16_t)c.dbits;
  } else {
    // byte m = code[2m] | code[2m+1] << 4.  Elements 2m and 2m+1 sit in the
    // adjacent lanes 2m and 2m+1 (m < 32, first element) or 2m-64 and 2m-63
    // (m >= 32, second element): an even lane e forms bytes e/2 and 32 + e/2
    // with its odd neighbour's codes, and a lane e = 4k joins them with lane
    // e + 2's into two 16-bit words, bytes 2k, 2k+1 and 32+2k, 33+2k.
    const uint32_t both = (uint32_t)(c.c0 | (c.c1 << 16));            // codes < 16
    const uint32_t pair = both | (lane_xor<1>(both, lane) << 4);      // even lanes
    const uint32_t quad = pair | (lane_xor<2>(pair, lane) << 8);      // lanes 4k
    if ((lane & 3) == 0) {
      *(uint16_t *)(dst + 2 + (lane >> 1)) = (uint16_t)(quad & 0xFFFFu);
      *(uint16_t *)(dst + 34 + (lane >> 1)) = (uint16_t)(quad >> 16);
    }
    if (lane == 0) *(uint16_t *)dst = (uint16_t)c.dbits;
  }
}

}  // namespace tbq4
