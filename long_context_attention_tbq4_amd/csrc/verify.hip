// TBQ4 multi-query verify attention (split-K) for gfx950.
//
// Page "Kontekst 262K na jednej RTX 4090: co dodałem do llama.cpp-turboq",
// section "Od czego zacząłem" (flash attention straight on TBQ4 blocks,
// dequantised in the inner loop, in the rotated domain) and the page's
// production configuration (--spec-type mtp --spec-draft-n-max 3): every
// decode step verifies the current token plus up to three drafted ones.
// Query i of a sequence sits at absolute position n_past + i and attends slots
// [0, n_past + i] -- causal among the drafted tokens, full over the prefix.
//
// Same streaming scheme as the decode split kernel (one wavefront per
// (sequence, KV head, split), 32-token tiles, K straight from registers, V
// transposed through LDS), but the K and V tiles are dequantised once for all
// n_q queries:
//   * the 16 MFMA columns hold (query, head) pairs -- queries 2c and 2c + 1
//     of column group c, G <= 8 heads each -- and one or two column groups
//     cover n_q <= 2 or n_q <= 4,
//   * q' is carried as an fp16 high part and the fp16 residual, multiplied
//     by the same K operand in two MFMAs that accumulate into one score; the
//     q' operands wait in LDS (one 16-byte slot per lane) instead of
//     registers, which keeps two wavefronts per SIMD for four queries,
//   * every column is a distinct (query, head), so each lane finishes its
//     own scores and P~ rows; P~ = p d^V is an fp16 value, rounded to
//     nearest, plus its fp16 residual, which a second MFMA multiplies by the
//     same V operand.
// Partial states use the decode workspace layout with (sequence, query) as
// the row index, so the decode merge kernel finishes them.
//
// K and V may each be stored as TBQ4 blocks, TBQ3 blocks, q8_0 rows or fp16
// rows (template arguments KF, VF); the fetch, operand and staging steps of
// each format are the decode kernel's.  q is rotated only when K is stored
// rotated, and the merge rotates the output back only when V is.
#include "tbq4_device.h"
#include "tbq4_launch.h"

#include <type_traits>

namespace tbq4 {

namespace {
constexpr int kTile = 32;
constexpr int kBlk = kTile / 16;
constexpr int kVRow = 80;           // staged TBQ4 V row: 64 index bytes + pad
constexpr int kE4Row = 144;         // staged TBQ3 V row: 128 e4m3 bytes + pad
constexpr int kF16Row = 288;        // staged fp16 V row: 256 bytes + pad
}  // namespace

template <typename QT, int CG, int KF, int VF>
__global__ __launch_bounds__(64) void verify_split_kernel(VerifyArgs a) {
  constexpr bool kKRot = KF == kFmtTbq4 || KF == kFmtTbq3;   // stored rotated
  constexpr uint32_t kKBytes = KF == kFmtTbq4 ? kBlockBytes : KF == kFmtTbq3 ? kBlockBytes3
                             : KF == kFmtQ8 ? kQ8RowBytes : 2 * kHeadDim;
  constexpr uint32_t kVBytes = VF == kFmtTbq4 ? kBlockBytes : VF == kFmtTbq3 ? kBlockBytes3
                             : VF == kFmtQ8 ? kQ8RowBytes : 2 * kHeadDim;
  __shared__ __attribute__((aligned(16))) uint8_t
      vlds[kTile * (VF == kFmtTbq4 ? kVRow : VF == kFmtF16 ? kF16Row : kE4Row)];
  __shared__ __attribute__((aligned(16))) float sk[kTile];
  __shared__ __attribute__((aligned(16))) float sv[kTile];
  // q8_0: one scale per (32-dim block, token), K scales times 2^-ex
  __shared__ __attribute__((aligned(16))) float skq[KF == kFmtQ8 ? 4 * kTile : 4];
  __shared__ __attribute__((aligned(16))) float svq[VF == kFmtQ8 ? 4 * kTile : 4];
  __shared__ __attribute__((aligned(16))) half8 qlds[CG][4][2][64];   // q' high / residual

  const int lane = threadIdx.x;
  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int G = a.group;
  const int quarter = lane >> 4;
  const int col = lane & 15;            // MFMA column: (query 2c + (col >> 3), head col & 7)
  const int head = col & 7;
  const int qsub = col >> 3;

  // ---------------- q' = R q * scale * log2(e) per (query, head) column
  float qv[CG][32];
  bool live[CG];
#pragma unroll
  for (int c = 0; c < CG; ++c) {
    const int qi = 2 * c + qsub;
    live[c] = qi < a.n_q && head < G;
    // lane quarter q holds dims 32 q + i; for a q8_0 K cache dims
    // 32 (i/8) + 8 q + i%8 instead, so that MFMA step k spans q8_0 block k.
    // A column past the drafted queries or the group reads query 0, head 0
    // (in bounds) and is zeroed below.
    const QT *qp = (const QT *)a.q +
                   (((size_t)b * a.n_q + (live[c] ? qi : 0)) * a.n_q_heads + (size_t)g * G +
                    (live[c] ? head : 0)) * kHeadDim;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      load_q8<QT>(qp + (KF == kFmtQ8 ? 32 * r + 8 * quarter : 32 * quarter + 8 * r), &qv[c][8 * r]);
    if constexpr (kKRot) {
      const uint32_t sw = a.sign[quarter];
#pragma unroll
      for (int i = 0; i < 32; ++i) qv[c][i] = ((sw >> i) & 1u) ? -qv[c][i] : qv[c][i];
#pragma unroll
      for (int h = 1; h < 32; h <<= 1)
#pragma unroll
        for (int i = 0; i < 32; ++i)
          if ((i & h) == 0) {
            const float x = qv[c][i], y = qv[c][i + h];
            qv[c][i] = x + y;
            qv[c][i + h] = x - y;
          }
      // dims 32 and 64 apart: lanes 16 and 32 apart
#pragma unroll
      for (int i = 0; i < 32; i += 2) butterfly_pair<16>(qv[c][i], qv[c][i + 1]);
#pragma unroll
      for (int i = 0; i < 32; i += 2) butterfly_pair<32>(qv[c][i], qv[c][i + 1]);
    }
  }
  // one power-of-two normalisation for all columns (the maximum of |v| f is
  // the maximum of |v| times f, rounded: rounding is monotonic)
  const float f = (kKRot ? 0.08838834764831845f : 1.0f) * a.qscale;
  float mx = 0.0f;
#pragma unroll
  for (int c = 0; c < CG; ++c)
#pragma unroll
    for (int i = 0; i < 32; ++i) mx = fmaxf(mx, fabsf(qv[c][i]));
  mx = fmaxf(mx, lane_xor_f32<1>(mx, lane));
  mx = fmaxf(mx, lane_xor_f32<2>(mx, lane));
  mx = fmaxf(mx, lane_xor_f32<4>(mx, lane));
  mx = fmaxf(mx, lane_xor_f32<8>(mx, lane));
  mx = fmaxf(mx, lane_xor_f32<16>(mx, lane));
  mx = fmaxf(mx, lane_xor_f32<32>(mx, lane));
  mx *= fabsf(f);
  int ex = 0;
  if (mx > 0.0f) { int e2; frexpf(mx, &e2); ex = 14 - e2; }
  ex = ex > 100 ? 100 : (ex < -100 ? -100 : ex);
  const float qs_inv = ldexpf(1.0f, -ex);
  const float fs = ldexpf(f, ex);   // f 2^ex: exact
#pragma unroll
  for (int c = 0; c < CG; ++c) {
    const float fc = live[c] ? fs : 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      // operand word j holds elements (8k + e0, 8k + e1): TBQ4 K operands
      // hold the 4 even then the 4 odd dims of a code word (pairs 0 2, 4 6,
      // 1 3, 5 7); TBQ3, fp16 and q8_0 K operands 8 consecutive elements of
      // the lane's order above
      u32x4 hw, lw;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int e0 = KF == kFmtTbq4 ? (j < 2 ? 4 * j : 4 * (j - 2) + 1) : 2 * j;
        const int e1 = KF == kFmtTbq4 ? e0 + 2 : e0 + 1;
        const float x0 = qv[c][8 * k + e0] * fc, x1 = qv[c][8 * k + e1] * fc;
        hw[j] = pk_f16(x0, x1);
        lw[j] = pk_f16_residual(hw[j], x0, x1);
      }
      qlds[c][k][0][lane] = __builtin_bit_cast(half8, hw);
      qlds[c][k][1][lane] = __builtin_bit_cast(half8, lw);
    }
  }

  // ---------------- token range: slots [0, n_past + n_q) in 32-token tiles
  const int n_kv = a.n_past + a.n_q;
  const int n_tiles = (n_kv + kTile - 1) / kTile;
  const int tiles_per_split = (n_tiles + a.n_splits - 1) / a.n_splits;
  const int t_begin = split * tiles_per_split;
  const int t_end = min(t_begin + tiles_per_split, n_tiles);

  const size_t row = ((size_t)b * a.n_kv_heads + g) * (size_t)a.capacity;
  const rsrc_t rk = make_rsrc(a.k + row * kKBytes, (uint32_t)a.capacity * kKBytes);
  const rsrc_t rv = make_rsrc(a.v + row * kVBytes, (uint32_t)a.capacity * kVBytes);

  float m_run[CG], l_run[CG];
  float4v o[CG][8];
#pragma unroll
  for (int c = 0; c < CG; ++c) {
    m_run[c] = -INFINITY;
    l_run[c] = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[c][i] = float4v{0.f, 0.f, 0.f, 0.f};
  }

  // transposed-read source addresses (fixed per lane): TBQ4 rows (index
  // bytes), TBQ3 rows (e4m3 bytes) and fp16 rows, as in the decode kernel
  int tr_off;
  {
    const int e = col >> 1;
    const int tok = 16 * (e >> 2) + 4 * quarter + (e & 3);
    tr_off = tok * kVRow + 8 * (col & 1);
  }
  int tr8_3_off;
  {
    const int j = col >> 1;
    const int tok = j < 4 ? 4 * quarter + j : 16 + 4 * quarter + (j - 4);
    tr8_3_off = tok * kE4Row + 8 * (col & 1);
  }
  const int tr16_off = (4 * quarter + (col >> 2)) * kF16Row + 8 * (col & 3);

  // raw fetch of one tile: per 16-token group this lane's 16 index bytes
  // (TBQ4: 5 words realigned by 0 or 2 bytes; TBQ3: 12 code bytes in one
  // 16-byte load) or its token's 32 fp16 dims (4 aligned 16-byte loads), and
  // the scales of token `lane`; a tile past the split reads as zeros
  // (q8_0 K: the lane's 8 codes of each of the token's 4 blocks in 10 words
  // and two of the token's block scales per lane; q8_0 V: the lane's block,
  // scale and 32 codes, in 9 words -- the decode kernel's fetches)
  constexpr int kKW = KF == kFmtF16 ? 4 : 1, kVW = VF == kFmtF16 ? 4 : VF == kFmtQ8 ? 2 : 1;
  struct Raw {
    u32x4 k4[kBlk * kKW], v4[kBlk * kVW];
    uint32_t k1[kBlk], v1[kBlk];
    u32x3 kq3[KF == kFmtQ8 ? 2 * kBlk : 1];
    u32x2 kq2[KF == kFmtQ8 ? 2 * kBlk : 1];
    uint16_t sk, sv;
    uint16_t skq[2];
  };
  const uint32_t lane_off = (uint32_t)col * kBlockBytes + 2 + 16 * quarter;
  const uint32_t shift = lane_off & 3u;   // (2 col + 2) mod 4: the same for TBQ3
  auto fetch = [&](Raw &r, int t) {
    const bool live = t < t_end;
    const uint32_t base = live ? (uint32_t)t * kTile * kBlockBytes : 0xFFFF0000u;
#pragma unroll
    for (int blk = 0; blk < kBlk; ++blk) {
      const uint32_t ad = (base + (uint32_t)(16 * blk) * kBlockBytes + lane_off) & ~3u;
      const uint32_t tok = (uint32_t)(t * kTile + 16 * blk + col);
      const uint32_t a3 = live ? (tok * kBlockBytes3 + 2u + 12u * quarter) & ~3u : 0xFFFF0000u;
      if constexpr (KF == kFmtTbq4) {
        r.k4[blk] = buf_load_x4(rk, ad);
        r.k1[blk] = buf_load_x1(rk, ad + 16);
      } else if constexpr (KF == kFmtTbq3) {
        r.k4[blk] = buf_load_x4(rk, a3);
      } else if constexpr (KF == kFmtQ8) {
        // codes 8 q .. 8 q + 7 of block c start at byte 34 c + 2 + 8 q of the
        // token (token rows are 8-byte aligned)
        const uint32_t tb = live ? tok * kQ8RowBytes + 8u * quarter : 0xFFFF0000u;
        r.kq3[2 * blk] = buf_load_x3(rk, tb);
        r.kq2[2 * blk] = buf_load_x2(rk, tb + 36);
        r.kq3[2 * blk + 1] = buf_load_x3(rk, tb + 68);
        r.kq2[2 * blk + 1] = buf_load_x2(rk, tb + 104);
      } else {
        const uint32_t fo = live ? tok * kKBytes + 64u * quarter : 0xFFFF0000u;
#pragma unroll
        for (int c = 0; c < 4; ++c) r.k4[4 * blk + c] = buf_load_x4(rk, fo + 16u * c);
      }
      if constexpr (VF == kFmtTbq4) {
        r.v4[blk] = buf_load_x4(rv, ad);
        r.v1[blk] = buf_load_x1(rv, ad + 16);
      } else if constexpr (VF == kFmtTbq3) {
        r.v4[blk] = buf_load_x4(rv, a3);
      } else if constexpr (VF == kFmtQ8) {
        const uint32_t vb = live ? (tok * kQ8RowBytes + 34u * quarter) & ~3u : 0xFFFF0000u;
        r.v4[2 * blk] = buf_load_x4(rv, vb);
        r.v4[2 * blk + 1] = buf_load_x4(rv, vb + 16);
        r.v1[blk] = buf_load_x1(rv, vb + 32);
      } else {
        const uint32_t fo = live ? tok * kVBytes + 64u * quarter : 0xFFFF0000u;
#pragma unroll
        for (int c = 0; c < 4; ++c) r.v4[4 * blk + c] = buf_load_x4(rv, fo + 16u * c);
      }
    }
    if constexpr (KF == kFmtQ8) {   // lane: token lane % 32, blocks 2 (lane / 32) + 0, 1
      const uint32_t so = live ? (uint32_t)(t * kTile + (lane & 31)) * kQ8RowBytes + 68u * (lane >> 5)
                               : 0xFFFF0000u;
      r.skq[0] = buf_load_u16(rk, so);
      r.skq[1] = buf_load_u16(rk, so + 34);
    }
    const uint32_t soff = lane < kTile ? base + (uint32_t)lane * kBlockBytes : 0xFFFF0000u;
    const uint32_t soff3 = lane < kTile && live ? (uint32_t)(t * kTile + lane) * kBlockBytes3 : 0xFFFF0000u;
    if constexpr (KF == kFmtTbq4) r.sk = buf_load_u16(rk, soff);
    if constexpr (KF == kFmtTbq3) r.sk = buf_load_u16(rk, soff3);
    if constexpr (VF == kFmtTbq4) r.sv = buf_load_u16(rv, soff);
    if constexpr (VF == kFmtTbq3) r.sv = buf_load_u16(rv, soff3);
  };

  // kPartial: the tile holds slots a draft query must not see (or slots past
  // the end); only the tiles at the end of the range
  auto process = [&](Raw &r, int t, auto partial_tag) {
    constexpr bool kPartial = decltype(partial_tag)::value;
    const int tok0 = t * kTile;
    uint32_t kw[kBlk][4];
    u32x4 kf[KF == kFmtF16 ? kBlk * 4 : 1];
    uint32_t kq[KF == kFmtQ8 ? kBlk : 1][8];
#pragma unroll
    for (int blk = 0; blk < kBlk; ++blk) {
      const u32x4 w = r.k4[blk];
      if constexpr (KF == kFmtQ8) {
        const u32x3 a0 = r.kq3[2 * blk], a2 = r.kq3[2 * blk + 1];
        const u32x2 a1 = r.kq2[2 * blk], a3 = r.kq2[2 * blk + 1];
        kq[blk][0] = alignbyte(a0[1], a0[0], 2u);
        kq[blk][1] = alignbyte(a0[2], a0[1], 2u);
        kq[blk][2] = a1[0];
        kq[blk][3] = a1[1];
        kq[blk][4] = alignbyte(a2[1], a2[0], 2u);
        kq[blk][5] = alignbyte(a2[2], a2[1], 2u);
        kq[blk][6] = a3[0];
        kq[blk][7] = a3[1];
      } else if constexpr (KF == kFmtTbq4) {
        kw[blk][0] = alignbyte(w[1], w[0], shift);
        kw[blk][1] = alignbyte(w[2], w[1], shift);
        kw[blk][2] = alignbyte(w[3], w[2], shift);
        kw[blk][3] = alignbyte(r.k1[blk], w[3], shift);
      } else if constexpr (KF == kFmtTbq3) {   // 96 code bits of the lane's 32 dims
        kw[blk][0] = alignbyte(w[1], w[0], shift);
        kw[blk][1] = alignbyte(w[2], w[1], shift);
        kw[blk][2] = alignbyte(w[3], w[2], shift);
      } else {
        // fp16 slots past the drafted tokens may hold anything: zero them
        const bool dead = kPartial && tok0 + 16 * blk + col >= n_kv;
#pragma unroll
        for (int c = 0; c < 4; ++c) kf[4 * blk + c] = dead ? u32x4{0u, 0u, 0u, 0u} : r.k4[4 * blk + c];
      }
    }
    __syncthreads();
#pragma unroll
    for (int blk = 0; blk < kBlk; ++blk) {
      if constexpr (VF == kFmtTbq4) {
        const u32x4 w = r.v4[blk];
        const u32x4 al = {alignbyte(w[1], w[0], shift), alignbyte(w[2], w[1], shift),
                          alignbyte(w[3], w[2], shift), alignbyte(r.v1[blk], w[3], shift)};
        *(u32x4 *)(vlds + (16 * blk + col) * kVRow + 16 * quarter) = al;
      } else if constexpr (VF == kFmtTbq3) {
        // the lane's 32 codes -> 32 e4m3 bytes (dims 32 quarter ..) in LDS
        const u32x4 w = r.v4[blk];
        const uint32_t w0 = alignbyte(w[1], w[0], shift), w1 = alignbyte(w[2], w[1], shift),
                       w2 = alignbyte(w[3], w[2], shift);
        uint32_t e[8];
#pragma unroll
        for (int c = 0; c < 4; ++c) tbq3_chunk_to_e4m3(tbq3_chunk(w0, w1, w2, c), e[2 * c], e[2 * c + 1]);
        uint8_t *rowp = vlds + (16 * blk + col) * kE4Row + 32 * quarter;
        *(u32x4 *)rowp = u32x4{e[0], e[1], e[2], e[3]};
        *(u32x4 *)(rowp + 16) = u32x4{e[4], e[5], e[6], e[7]};
      } else if constexpr (VF == kFmtQ8) {
        // block `quarter` of the token: scale then 32 codes, from byte 0 (even
        // quarter: codes 2 bytes into the words) or byte 2 (odd quarter)
        const u32x4 w0 = r.v4[2 * blk], w1 = r.v4[2 * blk + 1];
        const uint32_t d[9] = {w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3], r.v1[blk]};
        const bool odd = (quarter & 1) != 0;
        uint32_t cw[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) cw[j] = odd ? d[j + 1] : alignbyte(d[j + 1], d[j], 2u);
        uint8_t *rowp = vlds + (16 * blk + col) * kE4Row + 32 * quarter;
        *(u32x4 *)rowp = u32x4{cw[0], cw[1], cw[2], cw[3]};
        *(u32x4 *)(rowp + 16) = u32x4{cw[4], cw[5], cw[6], cw[7]};
        const uint16_t sbits = (uint16_t)(odd ? d[0] >> 16 : d[0] & 0xFFFFu);
        const bool dead = kPartial && tok0 + 16 * blk + col >= n_kv;   // (NaN guard)
        svq[quarter * kTile + 16 * blk + col] = dead ? 0.0f : half_bits_to_float(sbits);
      } else {
        const bool dead = kPartial && tok0 + 16 * blk + col >= n_kv;   // (as for K)
#pragma unroll
        for (int c = 0; c < 4; ++c)
          *(u32x4 *)(vlds + (16 * blk + col) * kF16Row + 64 * quarter + 16 * c) =
              dead ? u32x4{0u, 0u, 0u, 0u} : r.v4[4 * blk + c];
      }
    }
    if constexpr (KF == kFmtQ8) {
      const int tk = lane & 31, c0 = 2 * (lane >> 5);
      const bool dead = kPartial && tok0 + tk >= n_kv;
      skq[c0 * kTile + tk] = dead ? 0.0f : half_bits_to_float(r.skq[0]) * qs_inv;
      skq[(c0 + 1) * kTile + tk] = dead ? 0.0f : half_bits_to_float(r.skq[1]) * qs_inv;
    }
    if (lane < kTile) {
      float dk = qs_inv, dv = 1.0f;   // (q8_0: per-block scales above)
      if constexpr (KF == kFmtTbq4 || KF == kFmtTbq3) dk = half_bits_to_float(r.sk) * qs_inv;
      if constexpr (KF == kFmtQ8) dk = 1.0f;
      if constexpr (VF == kFmtTbq4 || VF == kFmtTbq3) dv = half_bits_to_float(r.sv);
      if constexpr (kPartial) {
        // slots past the drafted tokens may hold anything (NaN survives p = 0)
        if (tok0 + lane >= n_kv) dk = dv = 0.0f;
      }
      sk[lane] = dk;
      sv[lane] = dv;
    }
    // the decode kernel's lagged reference maximum: a tile rescales a column
    // group only when a score exceeds the reference by more than 8 (log2), so
    // p <= 256 and P~ = p d^V <= 65504 while every V scale is below 256; a
    // tile with a larger scale (or an unused slot's bits) uses lag 0
    bool vbig = VF == kFmtQ8;
    if constexpr (VF == kFmtTbq4 || VF == kFmtTbq3) vbig = __any(r.sv > 0x5BFFu);
    fetch(r, t + 1);

    // ---- scores: S^T[token][(query, head)] = K . (q'_hi + q'_lo)
    float4v acc[CG][kBlk];
    {
      half8 kh[kBlk][4];
#pragma unroll
      for (int blk = 0; blk < kBlk; ++blk)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          if constexpr (KF == kFmtTbq4) kh[blk][k] = word_to_half8(kw[blk][k]);
          else if constexpr (KF == kFmtTbq3)
            kh[blk][k] = tbq3_chunk_to_half8(tbq3_chunk(kw[blk][0], kw[blk][1], kw[blk][2], k));
          else if constexpr (KF == kFmtQ8) kh[blk][k] = i8x8_to_half8(kq[blk][2 * k], kq[blk][2 * k + 1]);
          else kh[blk][k] = __builtin_bit_cast(half8, kf[4 * blk + k]);
        }
      // consecutive MFMAs rotate through the CG x 2 accumulators, so none
      // waits for the one before it (each accumulator still takes step k's
      // high part, then its residual, in order)
#pragma unroll
      for (int c = 0; c < CG; ++c)
#pragma unroll
        for (int blk = 0; blk < kBlk; ++blk) acc[c][blk] = float4v{0.f, 0.f, 0.f, 0.f};
      if constexpr (KF == kFmtQ8) {
        // step k spans q8_0 block k, whose scale differs per token: each
        // step's product is taken alone and scaled in fp32
        __syncthreads();   // the block scales are staged
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          float4v st[CG][kBlk];
#pragma unroll
          for (int hl = 0; hl < 2; ++hl)
#pragma unroll
            for (int c = 0; c < CG; ++c) {
              const half8 qo = qlds[c][k][hl][lane];
#pragma unroll
              for (int blk = 0; blk < kBlk; ++blk)
                st[c][blk] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                    kh[blk][k], qo, hl ? st[c][blk] : float4v{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
            }
#pragma unroll
          for (int blk = 0; blk < kBlk; ++blk) {
            const float4v kd4 = *(const float4v *)(skq + k * kTile + 16 * blk + 4 * quarter);
#pragma unroll
            for (int c = 0; c < CG; ++c)
#pragma unroll
              for (int e = 0; e < 4; ++e) acc[c][blk][e] = fmaf(kd4[e], st[c][blk][e], acc[c][blk][e]);
          }
        }
      } else {
#pragma unroll
      for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int hl = 0; hl < 2; ++hl)
#pragma unroll
          for (int c = 0; c < CG; ++c) {
            const half8 qo = qlds[c][k][hl][lane];
#pragma unroll
            for (int blk = 0; blk < kBlk; ++blk)
              acc[c][blk] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kh[blk][k], qo, acc[c][blk], 0, 0, 0);
          }
      }
    }
    __syncthreads();

    half8 pa[CG], pr[CG];
    float pq[VF == kFmtQ8 ? CG : 1][8];   // q8_0 V: the weights p, scaled per block below
#pragma unroll
    for (int c = 0; c < CG; ++c) {
      const int qi = 2 * c + qsub;
      const float m_ref = m_run[c] == -INFINITY ? 0.0f : m_run[c];
      float t4[kBlk][4];
      float tmax = -INFINITY;
#pragma unroll
      for (int blk = 0; blk < kBlk; ++blk) {
        const float4v kd = *(const float4v *)(sk + 16 * blk + 4 * quarter);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          t4[blk][e] = fmaf(acc[c][blk][e], kd[e], -m_ref);
          if constexpr (kPartial)
            t4[blk][e] += (tok0 + 16 * blk + 4 * quarter + e <= a.n_past + qi) ? 0.0f : -INFINITY;
          tmax = fmaxf(tmax, t4[blk][e]);
        }
      }
      if (__any(tmax > (vbig ? 0.0f : 8.0f) || m_run[c] == -INFINITY)) {
        float smax = tmax + m_ref;
        smax = fmaxf(smax, __shfl_xor(smax, 16, 64));
        smax = fmaxf(smax, __shfl_xor(smax, 32, 64));
        const float m_new = fmaxf(m_run[c], smax);
        // a column that has seen no live slot yet keeps m = -inf: alpha 1
        const float alpha = m_new == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m_run[c] - m_new);
        m_run[c] = m_new;
        l_run[c] *= alpha;
        float al[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) al[e] = __shfl(alpha, 4 * quarter + e, 64);
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e) o[c][i][e] *= al[e];
        const float shift_t = m_new == -INFINITY ? 0.0f : m_ref - m_new;
#pragma unroll
        for (int blk = 0; blk < kBlk; ++blk)
#pragma unroll
          for (int e = 0; e < 4; ++e) t4[blk][e] += shift_t;
      }
      float psum = 0.0f;
      float pt[8];
#pragma unroll
      for (int blk = 0; blk < kBlk; ++blk) {
        const float4v vd = *(const float4v *)(sv + 16 * blk + 4 * quarter);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p = __builtin_amdgcn_exp2f(t4[blk][e]);
          psum += p;
          pt[4 * blk + e] = p * vd[e];
        }
      }
      l_run[c] += psum;
      if constexpr (VF == kFmtQ8) {
#pragma unroll
        for (int e = 0; e < 8; ++e) pq[c][e] = pt[e];   // (the staged token scales are 1)
      } else {
        uint32_t pw[4], rw[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          pw[j] = pk_f16(pt[2 * j], pt[2 * j + 1]);
          rw[j] = pk_f16_residual(pw[j], pt[2 * j], pt[2 * j + 1]);
        }
        pa[c] = __builtin_bit_cast(half8, u32x4{pw[0], pw[1], pw[2], pw[3]});
        pr[c] = __builtin_bit_cast(half8, u32x4{rw[0], rw[1], rw[2], rw[3]});
      }
    }

    // ---- O'^T += P~ V for every column group, then the residual of P~
    // times the same V operand (V dequantised once)
    if constexpr (VF == kFmtTbq4) {
#pragma unroll
      for (int cg = 0; cg < 4; ++cg) {
        typedef __attribute__((address_space(3))) int2v lds_i2;
        const int2v rr = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i2 *)(vlds + tr_off + 16 * cg));
        const uint32_t w0 = (uint32_t)rr[0], w1 = (uint32_t)rr[1];
        const half8 ve = lo_nibbles_to_half8(w0, w1);
        const half8 vo = lo_nibbles_to_half8(w0 >> 4, w1 >> 4);
#pragma unroll
        for (int c = 0; c < CG; ++c) {
          o[c][2 * cg] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa[c], ve, o[c][2 * cg], 0, 0, 0);
          o[c][2 * cg + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa[c], vo, o[c][2 * cg + 1], 0, 0, 0);
        }
#pragma unroll
        for (int c = 0; c < CG; ++c) {
          o[c][2 * cg] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pr[c], ve, o[c][2 * cg], 0, 0, 0);
          o[c][2 * cg + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pr[c], vo, o[c][2 * cg + 1], 0, 0, 0);
        }
      }
    } else if constexpr (VF == kFmtQ8) {
      // q8_0 V: codes staged as int8, one byte-transposed read per 16 dims;
      // dims 32 cc .. 32 cc + 31 lie in block cc, whose P~ is p times the
      // token's block-cc scale (value and residual)
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        half8 pb[CG], rb[CG];
        const float4v d0 = *(const float4v *)(svq + cc * kTile + 4 * quarter);
        const float4v d1 = *(const float4v *)(svq + cc * kTile + 16 + 4 * quarter);
#pragma unroll
        for (int c = 0; c < CG; ++c) {
          float pt[8];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            pt[e] = pq[c][e] * d0[e];
            pt[4 + e] = pq[c][4 + e] * d1[e];
          }
          uint32_t pw[4], rw[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            pw[j] = pk_f16(pt[2 * j], pt[2 * j + 1]);
            rw[j] = pk_f16_residual(pw[j], pt[2 * j], pt[2 * j + 1]);
          }
          pb[c] = __builtin_bit_cast(half8, u32x4{pw[0], pw[1], pw[2], pw[3]});
          rb[c] = __builtin_bit_cast(half8, u32x4{rw[0], rw[1], rw[2], rw[3]});
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int db = 2 * cc + h;
          typedef __attribute__((address_space(3))) int2v lds_i2;
          const int2v rr = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i2 *)(vlds + tr8_3_off + 16 * db));
          const half8 vv = i8x8_to_half8((uint32_t)rr[0], (uint32_t)rr[1]);
#pragma unroll
          for (int c = 0; c < CG; ++c) {
            o[c][db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pb[c], vv, o[c][db], 0, 0, 0);
            o[c][db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(rb[c], vv, o[c][db], 0, 0, 0);
          }
        }
      }
    } else {
      // TBQ3: e4m3 bytes, one byte-transposed read per 16 dims; fp16: two
      // 16-bit transposed reads per 16 dims (dim 16 db + col)
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        half8 vv;
        if constexpr (VF == kFmtTbq3) {
          typedef __attribute__((address_space(3))) int2v lds_i2;
          const int2v rr = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i2 *)(vlds + tr8_3_off + 16 * db));
          vv = e4m3x8_to_half8((uint32_t)rr[0], (uint32_t)rr[1]);
        } else {
          typedef __attribute__((address_space(3))) short4v lds_s4;
          const short4v r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4 *)(vlds + tr16_off + 32 * db));
          const short4v r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_s4 *)(vlds + tr16_off + 16 * kF16Row + 32 * db));
          const short8v s8 = {r0[0], r0[1], r0[2], r0[3], r1[0], r1[1], r1[2], r1[3]};
          vv = __builtin_bit_cast(half8, s8);
        }
#pragma unroll
        for (int c = 0; c < CG; ++c)
          o[c][db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa[c], vv, o[c][db], 0, 0, 0);
#pragma unroll
        for (int c = 0; c < CG; ++c)
          o[c][db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pr[c], vv, o[c][db], 0, 0, 0);
      }
    }
  };

  Raw r;
  fetch(r, t_begin);
  // tiles entirely at or below slot n_past are visible to every query
  const int t_full = min(t_end, (a.n_past + 1) / kTile);
  int t = t_begin;
  for (; t < t_full; ++t) process(r, t, std::false_type{});
  for (; t < t_end; ++t) process(r, t, std::true_type{});

  // ---------------- partial states: row (b * n_q + query) of the decode layout
  const int P = a.n_splits;
#pragma unroll
  for (int c = 0; c < CG; ++c) {
    l_run[c] += lane_xor_f32<16>(l_run[c], lane);
    l_run[c] += lane_xor_f32<32>(l_run[c], lane);
    const int qi = 2 * c + qsub;
    if (lane < 16 && qi < a.n_q && head < G) {
      float *w = a.ws + (((size_t)b * a.n_q + qi) * a.n_q_heads + (size_t)g * G + head) * P * 130 +
                 (size_t)split * 130;
      w[0] = m_run[c];
      w[1] = l_run[c];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int rc = 4 * quarter + e;          // P~ row = column (query, head)
      const int rq = 2 * c + (rc >> 3), rh = rc & 7;
      if (rq < a.n_q && rh < G) {
        float *dst = a.ws + (((size_t)b * a.n_q + rq) * a.n_q_heads + (size_t)g * G + rh) * P * 130 +
                     (size_t)split * 130 + 2;
        if constexpr (VF == kFmtTbq4) {
#pragma unroll
          for (int cg = 0; cg < 4; ++cg) {
            dst[32 * cg + 2 * col] = o[c][2 * cg][e];
            dst[32 * cg + 2 * col + 1] = o[c][2 * cg + 1][e];
          }
        } else {
#pragma unroll
          for (int db = 0; db < 8; ++db) dst[16 * db + col] = o[c][db][e];
        }
      }
    }
  }
}

hipError_t launch_verify_partial(const VerifyArgs &a, int batch, int q_dtype, hipStream_t stream) {
  dim3 grid(a.n_splits, a.n_kv_heads, batch);
  // (q dtype, column groups, K format, V format) -> kernel instance;
  // formats TBQ4 (0), fp16 (1), TBQ3 (2), q8_0 (3)
#define TBQ4_VF(QT, CG, KF, VF) reinterpret_cast<const void *>(&verify_split_kernel<QT, CG, KF, VF>)
#define TBQ4_VF_K(QT, CG, KF) \
  {TBQ4_VF(QT, CG, KF, 0), TBQ4_VF(QT, CG, KF, 1), TBQ4_VF(QT, CG, KF, 2), TBQ4_VF(QT, CG, KF, 3)}
#define TBQ4_VF_C(QT, CG) \
  {TBQ4_VF_K(QT, CG, 0), TBQ4_VF_K(QT, CG, 1), TBQ4_VF_K(QT, CG, 2), TBQ4_VF_K(QT, CG, 3)}
  static const void *const kernels[3][2][kNumFormats][kNumFormats] = {
                                                  {TBQ4_VF_C(float, 1), TBQ4_VF_C(float, 2)},
                                                  {TBQ4_VF_C(_Float16, 1), TBQ4_VF_C(_Float16, 2)},
                                                  {TBQ4_VF_C(uint16_t, 1), TBQ4_VF_C(uint16_t, 2)}};
#undef TBQ4_VF_C
#undef TBQ4_VF_K
#undef TBQ4_VF
  if (a.k_fmt < 0 || a.k_fmt >= kNumFormats || a.v_fmt < 0 || a.v_fmt >= kNumFormats)
    return hipErrorInvalidValue;
  if (q_dtype < 0 || q_dtype > 2) return hipErrorInvalidValue;
  const void *fn = kernels[q_dtype][a.n_q > 2 ? 1 : 0][a.k_fmt][a.v_fmt];
  VerifyArgs arg = a;
  void *params[] = {&arg};
  return hipLaunchKernel(fn, grid, dim3(64), params, 0, stream);
}

}  // namespace tbq4
