// TBQ4 prefill-chunk attention for gfx950.
//
// Page "Kontekst 262K na jednej RTX 4090: co dodałem do llama.cpp-turboq",
// section "Od czego zacząłem": flash attention reads raw TBQ4 blocks and
// dequantises them in its inner loop, in the rotated (Hadamard) domain, with
// no F16 buffer in memory.  A prefill chunk: query i of the chunk sits at
// absolute position n_past + i and attends keys 0 .. n_past + i.
//
// A workgroup owns one KV head and a tile of 256/G queries x G heads = 256
// rows (8 wavefronts x 32 rows, two per SIMD: the whole CU); blockIdx.x %
// n_kv_heads is the KV head, so on an 8-XCD part each XCD streams the cache
// of its own head.  Eight wavefronts share each staged tile, so a thread
// dequantises 16 codes of K and of V per tile and each tile is read by half
// as many workgroups as with four.  Per 64-key tile the workgroup
//   * fetches the next tile's packed K and V rows before it computes on the
//     current one (wavefront w loads eighth w of every key's index bytes;
//     together the eight cover the tile's contiguous bytes) and dequantises
//     them into the other half of a double-buffered LDS tile: fp16 codebook
//     values (K times the power of two 2^-ex that normalises q', applied by
//     the fp8 -> fp16 convert), and the key's two fp16 scales in one word,
//   * S^T = K Q'^T on v_mfma_f32_32x32x16_f16, with q' split into an fp16
//     high part and the fp16 residual that both accumulate into the same
//     fp32 scores (~22 bits of q'), then scales by d^K per key (a mixed
//     fp32 x fp16 multiply-add straight from the staged scale word),
//   * online softmax in the log2 domain, P~ = p d^V in fp16 (plus its fp16
//     residual as a second PV product in blocks where one key carries more
//     than 1/32 of a row's running weight),
//   * O'^T += V^T P~^T on v_mfma_f32_32x32x16_f16 with V^T read straight out
//     of the row-major LDS tile by ds_read_b64_tr_b16.
// The epilogue divides by the row sum, applies R^T and stores.
//
// LDS rows keep each 8-dimension group in nibble order (d0 d2 d4 d6 d1 d3 d5
// d7); q' uses the same order, and since the Walsh-Hadamard matrix is
// invariant under a permutation of index bits, the output transform runs in
// that order too, mapping positions back to dimensions only at the store.
#include "tbq4_device.h"
#include "tbq4_launch.h"

#include <type_traits>

namespace tbq4 {

constexpr int kKT = 64;             // keys per tile
// LDS row pitches.  K rows are read one row per lane (16 bytes): a 272-byte
// pitch (68 dwords) puts 8 consecutive rows on distinct banks.  V rows are
// read transposed, 4 consecutive rows x 32 bytes per 16 lanes: a 288-byte
// pitch (72 dwords) puts those on distinct banks, and the 16-byte chunks of
// rows with bit 2 set are swapped in pairs so that the stores of 8
// consecutive rows (one key per lane) do not collide either.
constexpr int kRowB = 272;
constexpr int kVRowB = 288;
constexpr int kTileB = kKT * kRowB;
constexpr int kVTileB = kKT * kVRowB;

// byte offset within V row r of the 16-byte chunk holding byte `byte`
__device__ __forceinline__ int v_swizzle(int r, int byte) { return byte ^ (((r >> 2) & 1) << 4); }

template <int KF, int VF> struct __attribute__((aligned(16))) PrefillLds {
  uint8_t k[2][kTileB];
  uint8_t v[2][kVTileB];
  // per key: the fp16 K scale in the low half, the fp16 V scale in the high
  uint32_t skv[2][kKT];
  // q8_0 tensors: one scale per (key, 32-dim block)
  float skq[KF == kFmtQ8 ? 2 : 1][4][KF == kFmtQ8 ? kKT : 4];
  float svq[VF == kFmtQ8 ? 2 : 1][4][VF == kFmtQ8 ? kKT : 4];
};

// dimension held at row position p (8-dimension groups in nibble order)
__device__ __forceinline__ int pos_to_dim(int p) {
  const int r = p & 7;
  return (p & ~7) | (r < 4 ? 2 * r : 2 * (r - 4) + 1);
}

template <typename T> __device__ __forceinline__ float ld(const T *p);
template <> __device__ __forceinline__ float ld<float>(const float *p) { return *p; }
template <> __device__ __forceinline__ float ld<_Float16>(const _Float16 *p) { return (float)*p; }
template <> __device__ __forceinline__ float ld<uint16_t>(const uint16_t *p) {   // bf16 bits
  return __uint_as_float((uint32_t)*p << 16);
}

// Cache formats (K and V independently): TBQ4 blocks (the path described
// above), TBQ3 blocks (50 bytes: scale + 3-bit codes), q8_0 rows (136 bytes:
// four blocks of an fp16 scale and 32 int8 codes, not rotated) or fp16 rows
// (256 bytes, not rotated).  Every format is staged into the same LDS tiles
// of fp16 values and per-key scales (q8_0: exact integer codes and one scale
// per key and 32-dim block, applied in fp32 after each block's K product and
// folded into the P~ of each 32-dim block of V); TBQ4 rows keep the nibble
// order, the others the natural dimension order, and q' and the epilogue
// follow the order of the tensor they meet.
template <int F> __device__ __forceinline__ int pos_to_dim_f(int p) {
  return F == kFmtTbq4 ? pos_to_dim(p) : p;
}
template <int F> constexpr uint32_t row_bytes_of() {
  return F == kFmtTbq4 ? kBlockBytes : F == kFmtTbq3 ? kBlockBytes3
       : F == kFmtQ8 ? kQ8RowBytes : 2 * kHeadDim;
}

// One thread's share of a tile fetch for one tensor: the 16 values at
// positions 16 fq .. 16 fq + 15 of key fkey -- TBQ4: 8 index bytes in 3 raw
// words (realigned by 0 or 2 bytes); TBQ3: 6 code bytes in 2 words; fp16: 32
// bytes; q8_0: 16 int8 codes of block fq / 2 in 5 words (realigned by 0 or
// 2 bytes) -- and the key's scale (threads with fq = 0; q8_0: the block's
// scale, threads with fq even).
template <int F> struct RawPart;
template <> struct RawPart<kFmtTbq4> { u32x3 w; uint16_t s; };
template <> struct RawPart<kFmtTbq3> { u32x2 w; uint16_t s; };
template <> struct RawPart<kFmtF16> { u32x4 w[2]; };
template <> struct RawPart<kFmtQ8> { u32x4 w; uint32_t w1; uint16_t s; };
template <int KF, int VF> struct TileRaw {
  RawPart<KF> k;
  RawPart<VF> v;
};

constexpr int kWaves = 8;           // wavefronts per workgroup (32 rows each)
// TBQ4 K and V read each 32-key block's MFMA operands ahead of their use (the
// other formats' staging holds more registers: there the same reads would
// spill, so they read each operand just before its MFMA)
template <int KF, int VF> constexpr bool kOpAheadOf = KF == kFmtTbq4 && VF == kFmtTbq4;
// A 32-key block takes the fp16 residual of P~ as a second PV product when one
// of its keys carries more than 1/kShareInv of a row's running weight sum.
constexpr float kShareInv = 32.0f;

template <typename QT, typename OT, int KF, int VF>
__global__ __launch_bounds__(64 * kWaves, 1) void prefill_kernel(PrefillArgs a) {
  __shared__ PrefillLds<KF, VF> L;
  __shared__ float q_wmax[kWaves];   // max |q'| per wavefront (the normalisation)
  constexpr bool kKRot = KF == kFmtTbq4 || KF == kFmtTbq3;   // stored rotated: q is rotated to meet it
  constexpr bool kVRot = VF == kFmtTbq4 || VF == kFmtTbq3;   // stored rotated: the output is rotated back
  constexpr bool kOpAhead = kOpAheadOf<KF, VF>;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int G = a.group;
  const int qpw = 32 / G;                        // queries per wavefront
  const int qpwg = kWaves * qpw;                 // queries per workgroup
  const int g = blockIdx.x % a.n_kv_heads;
  const int qt = blockIdx.x / a.n_kv_heads;
  const int b = blockIdx.y;

  const int row = lane & 31, half = lane >> 5;
  const int qi = qt * qpwg + wave * qpw + row / G;          // query index in the chunk
  const int hq = g * G + row % G;                           // query head
  const bool row_valid = qi < a.n_q;
  const int qi_c = row_valid ? qi : a.n_q - 1;
  const int key_limit = a.n_past + qi_c;                    // last key this row sees
  const int wave_q0 = min(qt * qpwg + wave * qpw, a.n_q - 1);
  const int wave_min_limit = a.n_past + wave_q0;            // smallest limit in the wave

  // ---------------- q' = R q * scale * log2(e): fp16 high part + residual
  // lane holds positions 16 c + 8 half + e (c = 0..7, e = 0..7)
  half8 qh[8], ql[8];
  float kscale;           // 2^-ex: staged TBQ K values carry it
  uint32_t kunit_bits;    // fp16 bits of 2^-ex
  {
    float x[64];
    const QT *qp = (const QT *)a.q + (((size_t)b * a.n_q + qi_c) * a.n_q_heads + hq) * kHeadDim;
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int d = pos_to_dim_f<KF>(16 * c + 8 * half + e);
        const float v = ld<QT>(qp + d);
        x[8 * c + e] = (kKRot && ((a.sign[d >> 5] >> (d & 31)) & 1u)) ? -v : v;
      }
    // Walsh-Hadamard over the 7 position bits: bits 0-2 = e, bit 3 = half
    // (lanes 32 apart), bits 4-6 = c
    if constexpr (kKRot) {
#pragma unroll
    for (int h = 1; h < 64; h <<= 1) {
#pragma unroll
      for (int i = 0; i < 64; ++i)
        if ((i & h) == 0) {
          const float u = x[i], w = x[i + h];
          x[i] = u + w;
          x[i + h] = u - w;
        }
    }
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      const float o = __shfl_xor(x[i], 32, 64);
      x[i] = half ? (o - x[i]) : (x[i] + o);
    }
    }
    const float f = (kKRot ? 0.08838834764831845f : 1.0f) * a.qscale;
    float mx = 0.0f;
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      x[i] *= f;
      mx = fmaxf(mx, fabsf(x[i]));
    }
    // one power-of-two normalisation for all rows of the workgroup: the
    // largest |q'| of its rows in [2^13, 2^14), with ex at most 11.  The
    // staged K values carry the factor back (codebook values times 2^-ex,
    // exact fp16 normals for -14 <= ex <= 11), so a score reaches log2 units
    // in the same fused multiply-add with d^K that subtracts the running
    // maximum.  (With ex at 11 the largest |q'| is at least 2^-4 of fp16's
    // largest power of two below its max; smaller elements keep 22-bit q'
    // pairs down to fp16's subnormal range, whose spacing is 2^-34 of the
    // largest |q'| or less.  ex is at least -14: q' entries stay below 2^28.)
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 1, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 2, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 4, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 8, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    if (lane == 0) q_wmax[wave] = mx;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mx = fmaxf(mx, q_wmax[w]);
    int ex = 0;
    if (mx > 0.0f) {
      int e2;
      frexpf(mx, &e2);
      ex = 14 - e2;
    }
    ex = ex > 11 ? 11 : (ex < -14 ? -14 : ex);
    kscale = ldexpf(1.0f, -ex);
    // K formats staged unscaled (fp16, q8_0) take 2^-ex as their key scale
    kunit_bits = (uint32_t)(15 - ex) << 10;
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float y = ldexpf(x[8 * c + e], ex);
        const _Float16 hi = (_Float16)y;
        qh[c][e] = hi;
        ql[c][e] = (_Float16)(y - (float)hi);
      }
  }

  const int q_last = min(qt * qpwg + qpwg, a.n_q) - 1;
  const int kv_end = a.n_past + q_last + 1;                  // keys the workgroup needs
  const int n_tiles = (kv_end + kKT - 1) / kKT;

  constexpr uint32_t kKB = row_bytes_of<KF>(), kVB = row_bytes_of<VF>();
  const size_t rowi = ((size_t)b * a.n_kv_heads + g) * (size_t)a.capacity;
  const rsrc_t rk = make_rsrc(a.k + rowi * kKB, (uint32_t)a.capacity * kKB);
  const rsrc_t rv = make_rsrc(a.v + rowi * kVB, (uint32_t)a.capacity * kVB);

  // fetch mapping: thread -> (key, sixteenth of its values), wavefront w
  // fetching values 16 w .. 16 w + 15 of the tile's 64 keys; packed start
  // offsets are even, so the realignment shift is 0 or 2 (per thread)
  const int fkey = tid & 63, fq = tid >> 6;
  const int n_keys = a.n_past + a.n_q;   // keys at or past this may hold anything
  // fetch one tensor's share of tile t (format F, buffer resource r)
  auto fetch_part = [&](auto &part, const rsrc_t &rs, int t, auto fmt_tag) {
    constexpr int F = decltype(fmt_tag)::value;
    const bool live = t * kKT + fkey < n_keys;
    if constexpr (F == kFmtTbq4) {
      const uint32_t base = (uint32_t)t * kKT * kBlockBytes;
      part.w = buf_load_x3(rs, (base + (uint32_t)fkey * kBlockBytes + 2 + 8 * fq) & ~3u);
      // a NaN scale of an unwritten slot must not survive the mask (p = 0)
      part.s = 0;
      if (fq == 0 && live) part.s = buf_load_u16(rs, base + (uint32_t)fkey * kBlockBytes);
    } else if constexpr (F == kFmtTbq3) {
      const uint32_t base = (uint32_t)t * kKT * kBlockBytes3;
      part.w = buf_load_x2(rs, (base + (uint32_t)fkey * kBlockBytes3 + 2 + 6 * fq) & ~3u);
      part.s = 0;
      if (fq == 0 && live) part.s = buf_load_u16(rs, base + (uint32_t)fkey * kBlockBytes3);
    } else if constexpr (F == kFmtQ8) {
      // codes 16 (fq & 1) .. + 15 of block fq / 2: byte 34 (fq / 2) + 2 +
      // 16 (fq & 1) of the key's 8-byte-aligned row
      const uint32_t kb = (uint32_t)(t * kKT + fkey) * kQ8RowBytes + 34u * (uint32_t)(fq >> 1);
      const uint32_t a4 = (kb + 2u + 16u * (uint32_t)(fq & 1)) & ~3u;
      part.w = buf_load_x4(rs, a4);
      part.w1 = buf_load_x1(rs, a4 + 16);
      part.s = 0;
      if ((fq & 1) == 0 && live) part.s = buf_load_u16(rs, kb);
    } else {
      // fp16 rows: an unwritten slot may hold NaN values, so it reads as zeros
      const uint32_t f = live ? (uint32_t)(t * kKT + fkey) * (2 * kHeadDim) + 32 * fq : 0xFFFF0000u;
      part.w[0] = buf_load_x4(rs, f);
      part.w[1] = buf_load_x4(rs, f + 16);
    }
  };
  auto fetch = [&](TileRaw<KF, VF> &r, int t) {
    fetch_part(r.k, rk, t, std::integral_constant<int, KF>{});
    fetch_part(r.v, rv, t, std::integral_constant<int, VF>{});
  };
  // the 16 fp16 values of a fetched share, in the tensor's position order,
  // as two 16-byte chunks; and the key's scale
  // (TBQ values times the power of two `sc`: 2^-ex for K, 1 for V)
  auto expand = [&](const auto &part, u32x4 &c0, u32x4 &c1, float sc, auto fmt_tag) {
    constexpr int F = decltype(fmt_tag)::value;
    if constexpr (F == kFmtTbq4) {
      const uint32_t sh = ((uint32_t)fkey * kBlockBytes + 2 + 8 * fq) & 3u;
      const uint32_t w0 = alignbyte(part.w[1], part.w[0], sh), w1 = alignbyte(part.w[2], part.w[1], sh);
      uint32_t r0, r1, r2, r3;
      nib4_to_f16(w0, r0, r1, sc);
      nib4_to_f16(w0 >> 4, r2, r3, sc);
      c0 = u32x4{r0, r1, r2, r3};
      nib4_to_f16(w1, r0, r1, sc);
      nib4_to_f16(w1 >> 4, r2, r3, sc);
      c1 = u32x4{r0, r1, r2, r3};
    } else if constexpr (F == kFmtTbq3) {
      // 16 codes = 48 bits from the (even) start byte
      const uint32_t sh = ((uint32_t)fkey * kBlockBytes3 + 2 + 6 * fq) & 3u;
      const uint32_t lo = alignbyte(part.w[1], part.w[0], sh);
      const uint32_t hi = part.w[1] >> (8 * sh);
      c0 = __builtin_bit_cast(u32x4, tbq3_chunk_to_half8(lo & 0xFFFFFFu, sc));
      c1 = __builtin_bit_cast(u32x4, tbq3_chunk_to_half8(((lo >> 24) | (hi << 8)) & 0xFFFFFFu, sc));
    } else if constexpr (F == kFmtQ8) {
      // int8 codes as exact fp16 values, natural order; the block scale is
      // applied per key after the products
      const uint32_t sh = ((uint32_t)fkey * kQ8RowBytes + 34u * (uint32_t)(fq >> 1) + 2u) & 3u;
      const u32x4 w = part.w;
      const uint32_t x0 = alignbyte(w[1], w[0], sh), x1 = alignbyte(w[2], w[1], sh);
      const uint32_t x2 = alignbyte(w[3], w[2], sh), x3 = alignbyte(part.w1, w[3], sh);
      c0 = __builtin_bit_cast(u32x4, i8x8_to_half8(x0, x1));
      c1 = __builtin_bit_cast(u32x4, i8x8_to_half8(x2, x3));
    } else {
      c0 = part.w[0];
      c1 = part.w[1];
    }
  };
  // fp16 bits of a key's scale (TBQ: the block's own, 0 for a slot past the
  // chunk; fp16 and q8_0: `unit`)
  auto scale_bits = [&](const auto &part, uint32_t unit, auto fmt_tag) -> uint32_t {
    constexpr int F = decltype(fmt_tag)::value;
    if constexpr (F == kFmtF16 || F == kFmtQ8) return unit;
    else return (uint32_t)part.s;
  };
  // dequantise a fetched share into LDS buffer `buf`: 16 fp16 values of K
  // and of V at row fkey, positions 16 fq .. 16 fq + 15
  auto stage = [&](const TileRaw<KF, VF> &r, int buf) {
    u32x4 c0, c1;
    expand(r.k, c0, c1, kscale, std::integral_constant<int, KF>{});
    uint8_t *kr = L.k[buf] + fkey * kRowB + 32 * fq;
    *(u32x4 *)kr = c0;
    *(u32x4 *)(kr + 16) = c1;
    expand(r.v, c0, c1, 1.0f, std::integral_constant<int, VF>{});
    uint8_t *vr = L.v[buf] + fkey * kVRowB;
    *(u32x4 *)(vr + v_swizzle(fkey, 32 * fq)) = c0;
    *(u32x4 *)(vr + v_swizzle(fkey, 32 * fq + 16)) = c1;
    if (fq == 0)
      L.skv[buf][fkey] = scale_bits(r.k, kunit_bits, std::integral_constant<int, KF>{}) |
                         scale_bits(r.v, 0x3C00u, std::integral_constant<int, VF>{}) << 16;
    // q8_0: the block scales (a slot at or past n_keys reads as scale 0, so
    // its finite codes contribute nothing)
    if constexpr (KF == kFmtQ8) {
      if ((fq & 1) == 0) L.skq[buf][fq >> 1][fkey] = half_bits_to_float(r.k.s);
    }
    if constexpr (VF == kFmtQ8) {
      if ((fq & 1) == 0) L.svq[buf][fq >> 1][fkey] = half_bits_to_float(r.v.s);
    }
  };

  float m_run = -INFINITY, l_run = 0.0f;
  float16v o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[i][e] = 0.0f;

  // transposed V reads: lane s of a 16-lane group points at key 4*half + s/4
  // (+ 8 for the second read) and position 16*((lane>>4)&1) + 4*(s&3)
  const int s16 = lane & 15;
  const int tr_row = 4 * half + (s16 >> 2);
  const int tr_col = 2 * (16 * ((lane >> 4) & 1) + 4 * (s16 & 3));

  {
    TileRaw<KF, VF> r0;
    fetch(r0, 0);
    stage(r0, 0);
  }
  __syncthreads();

  for (int kt = 0; kt < n_tiles; ++kt) {
    const int buf = kt & 1;
    const int key0 = kt * kKT;
    TileRaw<KF, VF> nxt;
    const bool more = kt + 1 < n_tiles;
    if (more) fetch(nxt, kt + 1);

    const uint8_t *kb = L.k[buf];
    const uint8_t *vb = L.v[buf];
    const bool masked = key0 + kKT - 1 > wave_min_limit;   // tile crosses the diagonal

#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int kb0 = 32 * sub;              // first key of this 32-key block in the tile
      // ---- S^T[key][row] = K (q'_hi + q'_lo)
      float16v sacc;
#pragma unroll
      for (int e = 0; e < 16; ++e) sacc[e] = 0.0f;
      if constexpr (KF == kFmtQ8) {
        // MFMA steps 2b and 2b + 1 span q8_0 block b, whose scale differs per
        // key: each block's product is taken alone and scaled in fp32
#pragma unroll
        for (int bq = 0; bq < 4; ++bq) {
          float16v t;
#pragma unroll
          for (int e = 0; e < 16; ++e) t[e] = 0.0f;
#pragma unroll
          for (int c = 2 * bq; c < 2 * bq + 2; ++c) {
            const half8 ka = *(const half8 *)(kb + (kb0 + row) * kRowB + 32 * c + 16 * half);
            t = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka, qh[c], t, 0, 0, 0);
            t = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka, ql[c], t, 0, 0, 0);
          }
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const float4v d4 = *(const float4v *)(&L.skq[buf][bq][kb0 + 8 * m + 4 * half]);
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2)
              sacc[4 * m + e2] = fmaf(d4[e2], t[4 * m + e2], sacc[4 * m + e2]);
          }
        }
      } else if constexpr (kOpAhead) {
        // all eight K operands are read before the first MFMA, so the chain
        // waits for LDS once rather than at every step
        half8 ka[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) ka[c] = *(const half8 *)(kb + (kb0 + row) * kRowB + 32 * c + 16 * half);
        __builtin_amdgcn_sched_barrier(0);   // (the scheduler would sink the reads)
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          sacc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka[c], qh[c], sacc, 0, 0, 0);
          sacc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka[c], ql[c], sacc, 0, 0, 0);
        }
      } else {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const half8 ka = *(const half8 *)(kb + (kb0 + row) * kRowB + 32 * c + 16 * half);
          sacc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka, qh[c], sacc, 0, 0, 0);
          sacc = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka, ql[c], sacc, 0, 0, 0);
        }
      }
      // the scale words of the lane's 16 keys are read while the MFMA chain
      // runs; for TBQ4 K and V the block's V^T operands follow (LDS reads
      // return in order, so the softmax waits for the scales only): their
      // latency passes under the softmax, and the residual pass reuses them
      u32x4 kv4[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) kv4[m] = *(const u32x4 *)(&L.skv[buf][kb0 + 8 * m + 4 * half]);
      typedef __attribute__((address_space(3))) short4v lds_s4;
      // V^T operand (ks, db) of this block: dims 32 db .., keys 16 ks ..
      auto v_operand = [&](int ks, int db) -> half8 {
        const int r0 = kb0 + 16 * ks + tr_row;     // (rows r0 and r0 + 8 share bit 2)
        const uint8_t *vbase = vb + r0 * kVRowB;
        const int col = v_swizzle(r0, tr_col + 64 * db);
        const short4v ra = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4 *)(vbase + col));
        const short4v rb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4 *)(vbase + 8 * kVRowB + col));
        return __builtin_bit_cast(half8, short8v{ra[0], ra[1], ra[2], ra[3], rb[0], rb[1], rb[2], rb[3]});
      };
      half8 vop[kOpAhead ? 2 : 1][4];
      if constexpr (kOpAhead) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int db = 0; db < 4; ++db) vop[ks][db] = v_operand(ks, db);
      }
      // the softmax issues at raised priority: the SIMD's other wavefront,
      // when it is in its MFMA phase, keeps the matrix core busy meanwhile
      __builtin_amdgcn_s_setprio(1);
      // element e holds key kb0 + 8 (e/4) + 4 half + e%4.  t = the score in
      // log2 units minus the reference m_ref (the row's running maximum, 0
      // before its first block): one fused multiply-add with the staged
      // fp16 d^K (the K values already carry 2^-ex).  Only a block that
      // raises some row's maximum (and the first block) moves the reference,
      // shifts t and rescales O' and l.
      const float m_ref = m_run == -INFINITY ? 0.0f : m_run;
      float t[16];
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) t[4 * m + e2] = fma_lo16(sacc[4 * m + e2], kv4[m][e2], -m_ref);
      if (masked) {
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2)
            t[4 * m + e2] += (key0 + kb0 + 8 * m + 4 * half + e2 <= key_limit) ? 0.0f : -INFINITY;
      }
      float tmax = -INFINITY;
#pragma unroll
      for (int e = 0; e < 16; ++e) tmax = fmaxf(tmax, t[e]);
      {   // the other half's maximum: one swap of the 32-lane halves leaves
          // the lower half's value in one result and the upper's in the other
        const auto hm = __builtin_amdgcn_permlane32_swap(__float_as_uint(tmax), __float_as_uint(tmax),
                                                         false, false);
        tmax = fmaxf(__uint_as_float(hm[0]), __uint_as_float(hm[1]));
      }
      float alpha = 1.0f;
      if (__any(tmax > 0.0f || m_run == -INFINITY)) {
        // (every row sees key 0, so a row's first block has a finite maximum;
        // a row with no key in this block keeps its reference: alpha 1)
        const float m_new = fmaxf(m_run, m_ref + tmax);
        alpha = __builtin_amdgcn_exp2f(m_run - m_new);   // 0 before the first block
        const float sh = m_ref - m_new;
#pragma unroll
        for (int e = 0; e < 16; ++e) t[e] += sh;
        tmax += sh;
        m_run = m_new;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int e = 0; e < 16; ++e) o[i][e] *= alpha;
      }
      float psum = 0.0f;
      float pt[16];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          const int e = 4 * m + e2;
          const float p = __builtin_amdgcn_exp2f(t[e]);
          psum += p;
          pt[e] = fma_hi16(p, kv4[m][e2], 0.0f);   // p d^V, rounded once
        }
      }
      l_run = l_run * alpha + psum;
      // A key whose weight is more than 1/kShareInv of the row's running sum
      // (this lane's half of it: a lower bound) makes the block take the
      // fp16 residual of P~ as a second PV product.  Keys below that share
      // enter with one fp16 rounding each, and those roundings average out
      // over the many keys that then carry the weight.
      const float p_top = __builtin_amdgcn_exp2f(tmax);
      const bool fine = __any(p_top * kShareInv > l_run);

      uint32_t pw[8], rw[8];
      if constexpr (VF != kFmtQ8) {
#pragma unroll
        for (int j = 0; j < 8; ++j) pw[j] = pk_f16(pt[2 * j], pt[2 * j + 1]);
        if (fine) {
#pragma unroll
          for (int j = 0; j < 8; ++j) rw[j] = pk_f16_residual(pw[j], pt[2 * j], pt[2 * j + 1]);
        }
      }

      __builtin_amdgcn_s_setprio(0);
      // ---- O'^T[dim][row] += V^T P~^T (then V^T times the residual of P~)
      auto pv = [&](const uint32_t *w) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const half8 pb = __builtin_bit_cast(half8, u32x4{w[4 * ks], w[4 * ks + 1], w[4 * ks + 2],
                                                           w[4 * ks + 3]});
#pragma unroll
          for (int db = 0; db < 4; ++db)
            o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kOpAhead ? vop[ks][db] : v_operand(ks, db), pb,
                                                           o[db], 0, 0, 0);
        }
      };
      if constexpr (VF == kFmtQ8) {
        // q8_0 V: dims 32 db .. 32 db + 31 form block db, whose P~ is p times
        // the key's block-db scale (the staged key scales are 1)
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          float q[16];
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const float4v d4 = *(const float4v *)(&L.svq[buf][db][kb0 + 8 * m + 4 * half]);
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) q[4 * m + e2] = pt[4 * m + e2] * d4[e2];
          }
          uint32_t w[8], x[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) w[j] = pk_f16(q[2 * j], q[2 * j + 1]);
          if (fine) {
#pragma unroll
            for (int j = 0; j < 8; ++j) x[j] = pk_f16_residual(w[j], q[2 * j], q[2 * j + 1]);
          }
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            const half8 vs = v_operand(ks, db);
            o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                vs, __builtin_bit_cast(half8, u32x4{w[4 * ks], w[4 * ks + 1], w[4 * ks + 2], w[4 * ks + 3]}),
                o[db], 0, 0, 0);
            if (fine)
              o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                  vs, __builtin_bit_cast(half8, u32x4{x[4 * ks], x[4 * ks + 1], x[4 * ks + 2], x[4 * ks + 3]}),
                  o[db], 0, 0, 0);
          }
        }
      } else {
        pv(pw);
        if (fine) pv(rw);
      }
    }

    if (more) stage(nxt, buf ^ 1);
    __syncthreads();
  }

  // ---------------- epilogue: normalise, o = R^T o', store
  l_run += __shfl_xor(l_run, 32, 64);
  const float inv = 1.0f / l_run;
  float y[64];       // index 16 db + e  <->  position 32 db + 8 (e/4) + 4 half + e%4
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) y[16 * db + e] = o[db][e] * inv;
  // position bits 0,1 = e bits 0,1; bits 3,4 = e bits 2,3; bits 5,6 = db
  if constexpr (kVRot) {
#pragma unroll
  for (int h = 1; h < 64; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 64; ++i)
      if ((i & h) == 0) {
        const float u = y[i], w = y[i + h];
        y[i] = u + w;
        y[i + h] = u - w;
      }
  }
#pragma unroll
  for (int i = 0; i < 64; ++i) {                 // position bit 2: lanes 32 apart
    const float t = __shfl_xor(y[i], 32, 64);
    y[i] = half ? (t - y[i]) : (y[i] + t);
  }
  }
  if (row_valid) {
    OT *dst = (OT *)a.out + (((size_t)b * a.n_q + qi) * a.n_q_heads + hq) * kHeadDim;
    const float r = kVRot ? 0.08838834764831845f : 1.0f;
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      const int db = i >> 4, e = i & 15;
      const int p = 32 * db + 8 * (e >> 2) + 4 * half + (e & 3);
      const int d = pos_to_dim_f<VF>(p);
      const float v = y[i] * r;
      dst[d] = (OT)((kVRot && ((a.sign[d >> 5] >> (d & 31)) & 1u)) ? -v : v);
    }
  }
}

hipError_t launch_prefill(const PrefillArgs &a, int batch, int q_dtype, int out_dtype,
                          hipStream_t stream) {
  const int qpwg = kWaves * (32 / a.group);
  const int n_qt = (a.n_q + qpwg - 1) / qpwg;
  const int64_t gx = (int64_t)n_qt * a.n_kv_heads;
  if (gx > 0x7FFFFFFF || batch > 65535) return hipErrorInvalidValue;
  dim3 grid((unsigned)gx, batch);
  // (q dtype, output dtype, K format, V format) -> kernel instance; formats
  // TBQ4 (0), fp16 (1), TBQ3 (2), q8_0 (3)
#define TBQ4_PF(QT, OT, KF, VF) reinterpret_cast<const void *>(&prefill_kernel<QT, OT, KF, VF>)
#define TBQ4_PF_K(QT, OT, KF) \
  {TBQ4_PF(QT, OT, KF, 0), TBQ4_PF(QT, OT, KF, 1), TBQ4_PF(QT, OT, KF, 2), TBQ4_PF(QT, OT, KF, 3)}
#define TBQ4_PF_Q(QT, OT) {TBQ4_PF_K(QT, OT, 0), TBQ4_PF_K(QT, OT, 1), TBQ4_PF_K(QT, OT, 2), \
                           TBQ4_PF_K(QT, OT, 3)}
  static const void *const kernels[3][2][kNumFormats][kNumFormats] = {
      {TBQ4_PF_Q(float, float), TBQ4_PF_Q(float, _Float16)},
      {TBQ4_PF_Q(_Float16, float), TBQ4_PF_Q(_Float16, _Float16)},
      {TBQ4_PF_Q(uint16_t, float), TBQ4_PF_Q(uint16_t, _Float16)}};
#undef TBQ4_PF_Q
#undef TBQ4_PF_K
#undef TBQ4_PF
  if (a.k_fmt < 0 || a.k_fmt >= kNumFormats || a.v_fmt < 0 || a.v_fmt >= kNumFormats)
    return hipErrorInvalidValue;
  if (q_dtype < 0 || q_dtype > 2) return hipErrorInvalidValue;
  const void *fn = kernels[q_dtype][out_dtype == 1 ? 1 : 0][a.k_fmt][a.v_fmt];
  PrefillArgs arg = a;
  void *params[] = {&arg};
  return hipLaunchKernel(fn, grid, dim3(64 * kWaves), params, 0, stream);
}

}  // namespace tbq4
