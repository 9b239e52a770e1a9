// Device-side helpers shared by the TBQ4 kernels (gfx950 / CDNA4 only).
//
// Block format (page "Kontekst 262K na jednej RTX 4090: co dodałem do
// llama.cpp-turboq", section "Od czego zacząłem"): 128 values -> 66 bytes, a
// binary16 scale d followed by 64 bytes of 4-bit codes (element 2j in the low
// nibble of byte 2+j).  A code is sign-magnitude, laid out like the 4-bit
// e2m1 float: bit 3 = sign, bits 0-2 = rank m of the magnitude in
//   0.125 0.375 0.625 0.9375 1.25 1.625 2 2.75
// Every level has four significant bits, so each is exact as an fp8 e4m3
// byte, as fp16 and as the integer 16*c; the kernels never form a dequantised
// tensor -- they turn codes into MFMA operands in registers or LDS and apply d
// once per token.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tbq4 {

constexpr int kHeadDim = 128;
constexpr int kBlockBytes = 66;

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef __fp16 fp16x2 __attribute__((ext_vector_type(2)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef float float16v __attribute__((ext_vector_type(16)));
typedef int int4v __attribute__((ext_vector_type(4)));
typedef int int16v __attribute__((ext_vector_type(16)));
typedef int int2v __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef short short8v __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------------------
// Codebook as byte tables for v_perm_b32 (a selector byte 0..3 picks a byte of
// the second source, 4..7 a byte of the first), indexed by the magnitude rank:
//   e4m3 bytes of the magnitudes: 20 2C 32 37 | 3A 3D 40 43 (sign = bit 7)
//   int8 16*c, positive: 2 6 10 15 | 20 26 32 44; negative: their negations
// ---------------------------------------------------------------------------
constexpr uint32_t kE4MagLo = 0x37322C20u, kE4MagHi = 0x43403D3Au;
constexpr uint32_t kI8PosLo = 0x0F0A0602u, kI8PosHi = 0x2C201A14u;
constexpr uint32_t kI8NegLo = 0xF1F6FAFEu, kI8NegHi = 0xD4E0E6ECu;

__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// Four codes, one in the low nibble of each byte of `t` (high nibbles are
// ignored) -> four e4m3 bytes: magnitude from the table, sign bit 3 -> bit 7.
__device__ __forceinline__ uint32_t nib4_to_e4m3(uint32_t t) {
  const uint32_t mag = perm(kE4MagHi, kE4MagLo, t & 0x07070707u);
  return mag | ((t << 4) & 0x80808080u);
}

// Four codes -> four fp16 codebook values (two fp16x2 words), each times
// `scale`, a power of two that the convert applies exactly (the caller keeps
// every product inside fp16's normal range).
__device__ __forceinline__ void nib4_to_f16(uint32_t t, uint32_t &w01, uint32_t &w23,
                                            float scale = 1.0f) {
  const uint32_t e = nib4_to_e4m3(t);
  fp16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(e, scale, false);
  fp16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(e, scale, true);
  w01 = __builtin_bit_cast(uint32_t, a);
  w23 = __builtin_bit_cast(uint32_t, b);
}

// One word of 8 codes (elements in nibble order 0..7) -> 8 fp16 values as an
// MFMA operand, in the order (n0 n2 n4 n6 n1 n3 n5 n7): low nibbles first.
__device__ __forceinline__ half8 word_to_half8(uint32_t w) {
  uint32_t r0, r1, r2, r3;
  nib4_to_f16(w, r0, r1);
  nib4_to_f16(w >> 4, r2, r3);
  u32x4 v = {r0, r1, r2, r3};
  return __builtin_bit_cast(half8, v);
}

// Low nibbles of two words (8 values) -> one half8 operand.
__device__ __forceinline__ half8 lo_nibbles_to_half8(uint32_t w0, uint32_t w1) {
  uint32_t r0, r1, r2, r3;
  nib4_to_f16(w0, r0, r1);
  nib4_to_f16(w1, r2, r3);
  u32x4 v = {r0, r1, r2, r3};
  return __builtin_bit_cast(half8, v);
}

// Four codes -> four int8 values 16*c: positive and negative tables looked up
// by rank, then byte i taken from the negative one when its sign bit is set.
__device__ __forceinline__ uint32_t nib4_to_i8(uint32_t t) {
  const uint32_t s7 = t & 0x07070707u;
  const uint32_t p = perm(kI8PosHi, kI8PosLo, s7);
  const uint32_t n = perm(kI8NegHi, kI8NegLo, s7);
  const uint32_t sel = ((t >> 1) & 0x04040404u) | 0x03020100u;
  return perm(n, p, sel);
}

// ---------------------------------------------------------------------------
// TBQ3 codes: 3-bit sign-magnitude (bit 2 = sign), magnitudes 0.25 0.75 1.375
// 2.25.  A 3-bit code is exactly a byte selector of v_perm over 8 table
// bytes, so the 8 signed values are one table:
//   e4m3 of +0.25 +0.75 +1.375 +2.25 | -0.25 -0.75 -1.375 -2.25
//          28    34    3B     41    | A8    B4    BB     C1
// ---------------------------------------------------------------------------
constexpr uint32_t kE4T3Lo = 0x413B3428u, kE4T3Hi = 0xC1BBB4A8u;

// Four 3-bit codes (bits 0..11 of y) -> one code in bits 0-2 of each byte:
// codes 0,1 stay in bits 0-5, codes 2,3 move to bits 16-21, then a copy
// shifted by 5 puts codes 1 and 3 at bits 8 and 24 (the other copies land
// in bits the mask clears).
__device__ __forceinline__ uint32_t spread3(uint32_t y) {
  const uint32_t z = (y & 0x3Fu) | (((y >> 6) & 0x3Fu) << 16);
  return (z | (z << 5)) & 0x07070707u;
}

// Eight 3-bit codes (bits 0..23 of x) -> eight e4m3 bytes in code order.
__device__ __forceinline__ void tbq3_chunk_to_e4m3(uint32_t x, uint32_t &e03, uint32_t &e47) {
  e03 = perm(kE4T3Hi, kE4T3Lo, spread3(x));
  e47 = perm(kE4T3Hi, kE4T3Lo, spread3(x >> 12));
}

// Eight 3-bit codes -> an fp16 MFMA operand, codes in natural order (each
// value times the power of two `scale`, as for nib4_to_f16).
__device__ __forceinline__ half8 tbq3_chunk_to_half8(uint32_t x, float scale = 1.0f) {
  uint32_t e03, e47;
  tbq3_chunk_to_e4m3(x, e03, e47);
  const fp16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(e03, scale, false);
  const fp16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(e03, scale, true);
  const fp16x2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(e47, scale, false);
  const fp16x2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(e47, scale, true);
  u32x4 v = {__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b),
             __builtin_bit_cast(uint32_t, c), __builtin_bit_cast(uint32_t, d)};
  return __builtin_bit_cast(half8, v);
}

// Eight e4m3 bytes (two words) -> an fp16 MFMA operand in byte order.
__device__ __forceinline__ half8 e4m3x8_to_half8(uint32_t w0, uint32_t w1) {
  const fp16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, false);
  const fp16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, true);
  const fp16x2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, false);
  const fp16x2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, true);
  u32x4 v = {__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b),
             __builtin_bit_cast(uint32_t, c), __builtin_bit_cast(uint32_t, d)};
  return __builtin_bit_cast(half8, v);
}

// Eight int8 values (two words, byte order) -> an fp16 MFMA operand.  Each
// byte b becomes the binary16 1024 + (b + 128) by a byte permute (0x64 is the
// high byte of 1024 and the flipped sign bit makes b + 128 unsigned), then
// 1152 is subtracted; exact, since every value is an integer below 2048.
__device__ __forceinline__ half8 i8x8_to_half8(uint32_t w0, uint32_t w1) {
  const uint32_t x0 = w0 ^ 0x80808080u, x1 = w1 ^ 0x80808080u;
  const fp16x2 k = {(_Float16)-1152.0f, (_Float16)-1152.0f};
  const fp16x2 a = __builtin_bit_cast(fp16x2, perm(0x64646464u, x0, 0x04010400u)) + k;
  const fp16x2 b = __builtin_bit_cast(fp16x2, perm(0x64646464u, x0, 0x04030402u)) + k;
  const fp16x2 c = __builtin_bit_cast(fp16x2, perm(0x64646464u, x1, 0x04010400u)) + k;
  const fp16x2 d = __builtin_bit_cast(fp16x2, perm(0x64646464u, x1, 0x04030402u)) + k;
  u32x4 v = {__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b),
             __builtin_bit_cast(uint32_t, c), __builtin_bit_cast(uint32_t, d)};
  return __builtin_bit_cast(half8, v);
}

// 24-bit chunk c (0..3) of a lane's 96 code bits held in three words.
__device__ __forceinline__ uint32_t tbq3_chunk(uint32_t w0, uint32_t w1, uint32_t w2, int c) {
  return c == 0 ? w0 : c == 1 ? __builtin_amdgcn_alignbit(w1, w0, 24)
                     : c == 2 ? __builtin_amdgcn_alignbit(w2, w1, 16) : (w2 >> 8);
}

// ---------------------------------------------------------------------------
// Buffer resources: loads through a V# are range checked by the hardware --
// bytes past num_records read as zero -- so a wave may over-fetch a few bytes
// at the end of a row without touching memory outside it.
// ---------------------------------------------------------------------------
typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t num_bytes) {
  // word 3 for CDNA: DST_SEL_XYZW + 32-bit data format, raw (untyped) access
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)num_bytes,
                                           0x00020000);
}

__device__ __forceinline__ u32x4 buf_load_x4(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
__device__ __forceinline__ u32x3 buf_load_x3(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x3, __builtin_amdgcn_raw_buffer_load_b96(r, off, 0, 0));
}
__device__ __forceinline__ u32x2 buf_load_x2(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
__device__ __forceinline__ uint32_t buf_load_x1(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
__device__ __forceinline__ uint16_t buf_load_u16(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}

__device__ __forceinline__ uint32_t alignbyte(uint32_t hi, uint32_t lo, uint32_t shift) {
  return __builtin_amdgcn_alignbyte(hi, lo, shift);
}

// Sixteen index bytes that start at byte offset `start` of a row (any even
// offset), as four little-endian words, from a 5-word aligned fetch.
__device__ __forceinline__ void load16_unaligned(rsrc_t r, uint32_t start, uint32_t out[4]) {
  const uint32_t a = start & ~3u;
  const u32x4 w = buf_load_x4(r, a);
  const uint32_t w4 = buf_load_x1(r, a + 16);
  const uint32_t s = start & 3u;
  out[0] = alignbyte(w[1], w[0], s);
  out[1] = alignbyte(w[2], w[1], s);
  out[2] = alignbyte(w[3], w[2], s);
  out[3] = alignbyte(w4, w[3], s);
}

// ---------------------------------------------------------------------------
// Weights carried as an fp16 value plus an fp16 residual.  P~ = p d^V enters
// the PV product as an fp16 MFMA operand; one fp16 rounding (relative 2^-11,
// the same for all 128 values of a V row) moves the output by up to 2^-11 of
// the V rows that carry the weight, which matters when few keys dominate.  The
// residual x - fp16(x) (exact in fp32) rounded to fp16 restores ~22 bits when
// it is accumulated by a second operand.  The residual is written out as
// instructions (v_fma_mix with the fp16 halves of the operand word as
// sources) so that it is taken from exactly the operand's bits: left to
// itself the compiler may round the exact product p d^V straight to fp16 for
// the residual while the operand holds the rounding of the fp32 product, two
// different numbers in the rare double-rounding cases.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t pk_f16(float x0, float x1) {
  return __builtin_bit_cast(uint32_t, fp16x2{(_Float16)x0, (_Float16)x1});
}
// fp16 pair of (x0 - h0, x1 - h1), h = the fp16 halves of the operand word hw
// (whichever way it was rounded), each difference rounded once
__device__ __forceinline__ uint32_t pk_f16_residual(uint32_t hw, float x0, float x1) {
  uint32_t rw;
  asm("v_fma_mixlo_f16 %0, %1, -1.0, %2 op_sel_hi:[1,0,0]" : "=v"(rw) : "v"(hw), "v"(x0));
  asm("v_fma_mixhi_f16 %0, %1, -1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]"
      : "+v"(rw) : "v"(hw), "v"(x1));
  return rw;
}

__device__ __forceinline__ float half_bits_to_float(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// a * h + c with h the fp16 in the low (fma_lo16) or high (fma_hi16) half of
// the word hw, widened exactly and fused in fp32 (one rounding): the same
// value as fmaf(a, (float)h, c), without a separate widening instruction.
__device__ __forceinline__ float fma_lo16(float a, uint32_t hw, float c) {
  float d;
  asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel_hi:[0,1,0]" : "=v"(d) : "v"(a), "v"(hw), "v"(c));
  return d;
}
__device__ __forceinline__ float fma_hi16(float a, uint32_t hw, float c) {
  float d;
  asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[0,1,0] op_sel_hi:[0,1,0]"
      : "=v"(d) : "v"(a), "v"(hw), "v"(c));
  return d;
}

// 16-lane row rotation by 8: lane j receives lane (j + 8) mod 16 of its row.
__device__ __forceinline__ float row_ror8(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                               0x128, 0xF, 0xF, true));
}

template <typename QT>
__device__ __forceinline__ float load_q(const QT *p);
template <> __device__ __forceinline__ float load_q<float>(const float *p) { return *p; }
template <> __device__ __forceinline__ float load_q<_Float16>(const _Float16 *p) { return (float)*p; }
// bf16 queries arrive as their 16-bit patterns: the upper half of an fp32
template <> __device__ __forceinline__ float load_q<uint16_t>(const uint16_t *p) {
  return __uint_as_float((uint32_t)*p << 16);
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
// x of lane (lane ^ H) for an fp32 value
template <int H> __device__ __forceinline__ float lane_xor_f32(float x, int lane) {
  return __uint_as_float(lane_xor<H>(__float_as_uint(x), lane));
}

// One butterfly level across lanes H apart (16: adjacent 16-lane rows, 32:
// the two halves) for two registers at once: lanes with bit H clear take
// x + x', the others x' - x (x' the partner lane's value).  The first swap
// puts a and its partner side by side in the rows (halves) of a with bit H
// clear and b and its partner in the others, so one add and one subtract
// form every result, and the second swap puts them back in place.
template <int H> __device__ __forceinline__ void butterfly_pair(float &a, float &b) {
  static_assert(H == 16 || H == 32, "butterfly_pair: rows or halves");
  const uint32_t ua = __float_as_uint(a), ub = __float_as_uint(b);
  const auto r = H == 16 ? __builtin_amdgcn_permlane16_swap(ua, ub, false, false)
                         : __builtin_amdgcn_permlane32_swap(ua, ub, false, false);
  const float x = __uint_as_float(r[0]), y = __uint_as_float(r[1]);
  const float s = x + y, d = x - y;
  const auto t = H == 16 ? __builtin_amdgcn_permlane16_swap(__float_as_uint(s), __float_as_uint(d), false, false)
                         : __builtin_amdgcn_permlane32_swap(__float_as_uint(s), __float_as_uint(d), false, false);
  a = __uint_as_float(t[0]);
  b = __uint_as_float(t[1]);
}

// Eight consecutive query elements from a 16-byte aligned address, as fp32.
template <typename QT> __device__ __forceinline__ void load_q8(const QT *p, float *x);
template <> __device__ __forceinline__ void load_q8<float>(const float *p, float *x) {
  const float4v a = *(const float4v *)p, b = *(const float4v *)(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[i] = a[i];
    x[4 + i] = b[i];
  }
}
template <> __device__ __forceinline__ void load_q8<_Float16>(const _Float16 *p, float *x) {
  const half8 h = *(const half8 *)p;
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = (float)h[i];
}
template <> __device__ __forceinline__ void load_q8<uint16_t>(const uint16_t *p, float *x) {
  const u32x4 w = *(const u32x4 *)p;   // bf16 pairs: the upper halves of fp32s
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}

}  // namespace tbq4
