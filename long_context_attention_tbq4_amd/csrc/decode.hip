// TBQ4 split-K decode attention for gfx950.
//
// Page "Kontekst 262K na jednej RTX 4090: co dodałem do llama.cpp-turboq",
// section "Od czego zacząłem": the flash-attention kernel reads raw TBQ4
// blocks from global memory and dequantises them in its inner loop, in the
// rotated (Hadamard) domain, so there is no dequantisation pass and no F16
// buffer.  Rotated-domain attention: q' = R q, s_j = scale d^K_j (q' . c^K_j),
// o' = sum_j p_j d^V_j c^V_j, o = R^T o' (R orthogonal).
//
// Work split (flash decoding): one wavefront per (sequence, KV head, split)
// streams a contiguous run of 32-token tiles and writes a partial softmax
// state (m, l, o'[128]) for each of the G query heads of that KV head; a
// second kernel merges the splits, normalises, applies R^T and stores.
//
// Per 32-token tile a wavefront
//   * fetches 2 x 16 tokens of K and V with 16-byte-per-lane buffer loads
//     (lane = token x 32-dimension quarter; a 16-token group is one
//     contiguous 1056-byte run, so every fetched line is fully used),
//   * S^T = K Q'^T on v_mfma_f32_16x16x32_f16: K nibbles go straight from
//     registers to fp16 operands (byte-permute LUT -> e4m3 -> fp16); the 16
//     MFMA columns hold the G <= 8 query heads twice, as an fp16 high part
//     and the fp16 residual, so the scores carry ~22 bits of q,
//   * finishes each (head, token) score once: the lanes of MFMA columns 0-7
//     take the first 16-token block, those of columns 8-15 the second,
//   * stages the V index bytes in LDS and reads them back transposed with
//     ds_read_b64_tr_b8 (8 tokens x 1 byte per lane), dequantises them the
//     same way and runs O'^T += P~ V on MFMA, with P~ = p d^V as an fp16
//     value (rows 0-7 of the P~ operand) plus its fp16 residual (rows 8-15),
//   * keeps the online-softmax state in the log2 domain.
#include "tbq4_device.h"
#include "tbq4_launch.h"
#include "tbq4_quant.h"

#include <hip/hip_ext.h>
#include <mutex>
#include <type_traits>

namespace tbq4 {

constexpr int kTile = kDecodeTile;  // tokens per loop iteration
constexpr int kBlk = kTile / 16;    // 16-token MFMA row blocks per tile
constexpr int kVRow = 80;           // LDS bytes per staged V row (64 + pad)

// Cache formats of the K and V tensors (template arguments KF, VF): TBQ4
// blocks (the path described above), fp16 rows (not rotated), TBQ3 blocks or
// q8_0 rows (not rotated); each format's fetch, operand and staging steps
// sit beside the TBQ4 ones below.  q is rotated when K is a TBQ format; the
// merge applies R^T when V is.
constexpr int kE4Row = 144;         // LDS bytes per staged TBQ3 (e4m3) or q8_0 (int8) V row: 128 bytes + pad
                                    // (36 dwords: the 8 rows of one byte-transposed read
                                    // fall on distinct banks)
constexpr int kF16Row = 288;        // LDS bytes per staged fp16 V row (256 + pad; 72 dwords
                                    // put the 4 rows of one transposed read on distinct banks)

// Word of the P~ operand for two weights (x0, x1) of a head: lanes 0-7 of
// each 16-lane row get the fp16 pair nearest (x0, x1); lanes 8-15, whose own
// weights are zero, get the fp16 pair of what that rounding left out in the
// lane 8 below.
__device__ __forceinline__ uint32_t split_f16x2(float x0, float x1) {
  const uint32_t hw = pk_f16(x0, x1);
  const int rw = (int)pk_f16_residual(hw, x0, x1);
  return hw | (uint32_t)__builtin_amdgcn_update_dpp(0, rw, 0x128, 0xF, 0xF, true);
}

// Level magnitude of a TBQ4 (bits 0-2) or TBQ3 (bits 0-1) code, signed by
// its top bit: exact dyadic values.
template <int FMT> __device__ __forceinline__ double code_level(int c) {
  if constexpr (FMT == kFmtTbq3) {
    const double mag = (c & 3) == 0 ? 0.25 : (c & 3) == 1 ? 0.75 : (c & 3) == 2 ? 1.375 : 2.25;
    return (c & 4) ? -mag : mag;
  } else {
    constexpr double kMag[8] = {0.125, 0.375, 0.625, 0.9375, 1.25, 1.625, 2.0, 2.75};
    const double mag = kMag[c & 7];
    return (c & 8) ? -mag : mag;
  }
}

// element i of a head vector of dtype 0 (fp32), 1 (fp16) or 2 (bf16), exact in fp64
__device__ __forceinline__ double load_any(const void *row, int dtype, int i) {
  if (dtype == 0) return load_exact<float>((const float *)row + i);
  if (dtype == 1) return load_exact<_Float16>((const _Float16 *)row + i);
  return load_exact<uint16_t>((const uint16_t *)row + i);
}
template <int FMT>
__device__ __forceinline__ LaneCodes quantize_any(const void *row, int dtype, uint32_t w_a,
                                                  uint32_t w_b, int lane) {
  return quantize_values<FMT>(load_any(row, dtype, lane), load_any(row, dtype, lane + 64), w_a,
                              w_b, lane);
}

// The new token of a decode step, two wavefronts per (sequence b, KV head g),
// which each quantise one of its head vectors with the append kernel's
// arithmetic (identical bytes) and store it at the token's slot, and between
// them write the token's own partial state for the G query heads of g as
// split n_splits - 1:
//   K wavefront: m = qscale * (q . k~), l = 1, with k~ = R^T (d^K level(code^K))
//                (the dequantised key, rotated back in fp32);
//   V wavefront: o' = d^V level(code^V) (rotated domain, as the splits keep it).
// The streaming splits never read the token (they stop at its slot), so the
// stores and the partial state need no ordering against them; the merge, a
// later launch, sees them.  Splitting the work halves what each wavefront
// takes from the vector unit of the SIMD it shares with two streaming
// wavefronts.
template <typename QT, int KF, int VF>
__device__ void step_new_token(const DecodeArgs &a, int b, int g, int is_v, int lane) {
  constexpr uint32_t kKB = KF == kFmtTbq3 ? kBlockBytes3 : kBlockBytes;
  constexpr uint32_t kVB = VF == kFmtTbq3 ? kBlockBytes3 : kBlockBytes;
  const int G = a.group, P = a.n_splits;
  float *wsb = a.ws + ((size_t)b * a.n_q_heads + (size_t)g * G) * P * 130 + (size_t)(P - 1) * 130;
  const int slot = a.ctx_lens ? a.ctx_lens[b] : a.n_ctx;
  const bool none = slot < 0 || slot > a.n_ctx;   // no token for this sequence: an empty state
  const size_t vec = (size_t)b * a.n_kv_heads + g;   // source row and cache row
  const size_t at = vec * (size_t)a.capacity + (size_t)(none ? 0 : slot);
  const uint32_t w_a = lane < 32 ? a.sign[0] : a.sign[1];
  const uint32_t w_b = lane < 32 ? a.sign[2] : a.sign[3];
  const size_t src = vec * kHeadDim * (a.new_dtype == 0 ? 4 : 2);
  if (is_v) {
    float o0 = 0.0f, o1 = 0.0f;
    if (!none) {
      const LaneCodes vc = quantize_any<VF>((const uint8_t *)a.v_new + src, a.new_dtype, w_a, w_b,
                                            lane);
      // the caches are the caller's writable buffers (held const for the streaming splits)
      store_lanes<VF>(const_cast<uint8_t *>(a.v) + at * kVB, vc, lane);
      const double dv = half_value(vc.dbits);
      o0 = (float)(dv * code_level<VF>(vc.c0));   // exact: <= 15 significant bits
      o1 = (float)(dv * code_level<VF>(vc.c1));
    }
    for (int h = 0; h < G; ++h) {
      float *w = wsb + (size_t)h * P * 130;
      w[2 + lane] = o0;
      w[66 + lane] = o1;
    }
    return;
  }
  if (none) {
    for (int h = 0; h < G; ++h) {
      if (lane == 0) {
        float *w = wsb + (size_t)h * P * 130;
        w[0] = -INFINITY;
        w[1] = 0.0f;
      }
    }
    return;
  }
  // the queries' two values per lane, loaded before the quantiser runs
  const QT *qb = (const QT *)a.q + ((size_t)b * a.n_q_heads + (size_t)g * G) * kHeadDim;
  float qa[8], qc[8];
#pragma unroll
  for (int h = 0; h < 8; ++h) {
    qa[h] = h < G ? load_q<QT>(qb + (size_t)h * kHeadDim + lane) : 0.0f;
    qc[h] = h < G ? load_q<QT>(qb + (size_t)h * kHeadDim + lane + 64) : 0.0f;
  }
  const LaneCodes kc = quantize_any<KF>((const uint8_t *)a.k_new + src, a.new_dtype, w_a, w_b,
                                        lane);
  store_lanes<KF>(const_cast<uint8_t *>(a.k) + at * kKB, kc, lane);
  // k~ = s * (H k') / sqrt(128), elements lane and lane + 64, in fp32
  const float dk = (float)half_value(kc.dbits);
  float k0 = dk * (float)code_level<KF>(kc.c0), k1 = dk * (float)code_level<KF>(kc.c1);
#pragma unroll
  for (int hh = 1; hh < 64; hh <<= 1) {
    float p0, p1;
    switch (hh) {
      case 1: p0 = lane_xor_f32<1>(k0, lane); p1 = lane_xor_f32<1>(k1, lane); break;
      case 2: p0 = lane_xor_f32<2>(k0, lane); p1 = lane_xor_f32<2>(k1, lane); break;
      case 4: p0 = lane_xor_f32<4>(k0, lane); p1 = lane_xor_f32<4>(k1, lane); break;
      case 8: p0 = lane_xor_f32<8>(k0, lane); p1 = lane_xor_f32<8>(k1, lane); break;
      case 16: p0 = lane_xor_f32<16>(k0, lane); p1 = lane_xor_f32<16>(k1, lane); break;
      default: p0 = lane_xor_f32<32>(k0, lane); p1 = lane_xor_f32<32>(k1, lane); break;
    }
    const bool upper = (lane & hh) != 0;
    k0 = upper ? (p0 - k0) : (k0 + p0);
    k1 = upper ? (p1 - k1) : (k1 + p1);
  }
  {
    const float x = k0, y = k1;
    k0 = x + y;
    k1 = x - y;
  }
  const float r = 0.08838834764831845f;
  k0 = ((w_a >> (lane & 31)) & 1u) ? -(k0 * r) : k0 * r;
  k1 = ((w_b >> (lane & 31)) & 1u) ? -(k1 * r) : k1 * r;
  float sc[8];
#pragma unroll
  for (int h = 0; h < 8; ++h) sc[h] = fmaf(qa[h], k0, qc[h] * k1);
#pragma unroll
  for (int h = 0; h < 8; ++h) {
    sc[h] += lane_xor_f32<32>(sc[h], lane);
    sc[h] += lane_xor_f32<16>(sc[h], lane);
    sc[h] += lane_xor_f32<8>(sc[h], lane);
    sc[h] += lane_xor_f32<4>(sc[h], lane);
    sc[h] += lane_xor_f32<2>(sc[h], lane);
    sc[h] += lane_xor_f32<1>(sc[h], lane);
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < 8; ++h) {
      if (h < G) {
        float *w = wsb + (size_t)h * P * 130;
        w[0] = sc[h] * a.qscale;
        w[1] = 1.0f;
      }
    }
  }
}

template <typename QT, int KF, int VF>
__global__ __launch_bounds__(64) void decode_split_kernel(DecodeArgs a) {
  // bytes per head vector of each tensor
  constexpr uint32_t kKBytes = KF == kFmtTbq4 ? kBlockBytes : KF == kFmtTbq3 ? kBlockBytes3
                             : KF == kFmtQ8 ? kQ8RowBytes : 2 * kHeadDim;
  constexpr uint32_t kVBytes = VF == kFmtTbq4 ? kBlockBytes : VF == kFmtTbq3 ? kBlockBytes3
                             : VF == kFmtQ8 ? kQ8RowBytes : 2 * kHeadDim;
  constexpr bool kKRot = KF == kFmtTbq4 || KF == kFmtTbq3;   // stored rotated
  __shared__ __attribute__((aligned(16))) uint8_t
      vlds[kTile * (VF == kFmtTbq4 ? kVRow : VF == kFmtF16 ? kF16Row : kE4Row)];
  // q8_0: one scale per (32-dim block, token): K scales * 2^-ex, V scales
  // followed by 32 zeros (read by the lanes of P~ rows 8-15)
  __shared__ __attribute__((aligned(16))) float skq[KF == kFmtQ8 ? 4 * kTile : 4];
  __shared__ __attribute__((aligned(16))) float svq[VF == kFmtQ8 ? 4 * kTile + 32 : 4];
  __shared__ __attribute__((aligned(16))) float sk[kTile];   // d^K * 2^-ex per token
  __shared__ __attribute__((aligned(16))) float sv[kTile + 32];   // d^V per token, then zeros

  const int lane = threadIdx.x;
  int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  if constexpr ((KF == kFmtTbq4 || KF == kFmtTbq3) && (VF == kFmtTbq4 || VF == kFmtTbq3)) {
    if (a.step) {
      // decode step: a 1-D grid of the streaming splits in (split, head,
      // sequence) order -- the order and XCD placement of the plain 3-D grid
      // -- followed by two new-token wavefronts per (head, sequence).  The
      // new-token wavefronts come last so that the dispatcher has already
      // given every SIMD its share of streaming wavefronts when they arrive.
      const int n_stream = a.n_splits - 1;
      const int L = blockIdx.x;
      const int rows = (int)gridDim.x / (n_stream + 2);   // n_kv_heads * batch
      if (L >= n_stream * rows) {   // the new token: K then V wavefront of each row
        const int e = L - n_stream * rows, r = e >> 1;
        step_new_token<QT, KF, VF>(a, r / a.n_kv_heads, r % a.n_kv_heads, e & 1, lane);
        return;
      }
      split = L % n_stream;
      g = (L / n_stream) % a.n_kv_heads;
      b = L / (n_stream * a.n_kv_heads);
    }
  }
  const int G = a.group;
  const int quarter = lane >> 4;       // 32-dimension quarter / token sub-group
  const int col = lane & 15;           // MFMA column: query head (col & 7), part col >> 3
  const int head = col & 7;
  const bool lo_part = col >= 8;
  static_assert(kBlk == 2, "the score split between lanes 0-7 and 8-15 pairs two blocks");
  // lanes of P~ rows 8-15 read zero V scales (their rows carry the residual
  // of rows 0-7, moved in from lanes 0-7)
  const float *sv_rd = lo_part ? sv + kTile : sv;
  if (lane < 32) sv[kTile + lane] = 0.0f;
  if constexpr (VF == kFmtQ8) {
    if (lane < 32) svq[4 * kTile + lane] = 0.0f;
  }

  // ---------------- token range of this split: this sequence's length (from
  // device memory when given) in 32-token tiles, spread evenly over the splits
  // (a decode step: the slots before the new token's, none when its slot is
  // outside [0, n_ctx]; the last split index is the new token's)
  int n_ctx = a.n_ctx;
  if (a.ctx_lens) {
    const int len = a.ctx_lens[b];
    n_ctx = a.step && (len < 0 || len > a.n_ctx) ? 0 : min(max(len, 0), a.n_ctx);
  }
  const int n_stream = a.n_splits - a.step;
  const int n_tiles = (n_ctx + kTile - 1) / kTile;
  const int tiles_per_split = (n_tiles + n_stream - 1) / n_stream;
  const int t_begin = split * tiles_per_split;
  const int t_end = min(t_begin + tiles_per_split, n_tiles);

  const size_t row = ((size_t)b * a.n_kv_heads + g) * (size_t)a.capacity;
  const rsrc_t rk = make_rsrc(a.k + row * kKBytes, (uint32_t)a.capacity * kKBytes);
  const rsrc_t rv = make_rsrc(a.v + row * kVBytes, (uint32_t)a.capacity * kVBytes);

  float m_run = -INFINITY, l_run = 0.0f;
  float4v o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = float4v{0.f, 0.f, 0.f, 0.f};

  // transposed-read source address (fixed per lane): lane s of 16-lane group
  // G4 points at token tau(G4, s/2), byte 8*(s&1) of a 16-byte column group
  int tr_off;
  {
    const int e = col >> 1;
    const int tok = 16 * (e >> 2) + 4 * quarter + (e & 3);
    tr_off = tok * kVRow + 8 * (col & 1);
  }
  const int tr16_off = (4 * quarter + (col >> 2)) * kF16Row + 8 * (col & 3);
  // TBQ3 V (e4m3 rows): source lane s of a 16-lane group points at the
  // token of P~ operand position 8 quarter + s/2 and bytes 8 (s & 1) .. + 7
  // of a 16-dim block, so a byte-transposed read gives a lane 8 tokens of
  // dim 16 db + col
  int tr8_3_off;
  {
    const int j = col >> 1;
    const int tok = j < 4 ? 4 * quarter + j : 16 + 4 * quarter + (j - 4);
    tr8_3_off = tok * kE4Row + 8 * (col & 1);
  }

  // Raw fetch of one 32-token tile: per 16-token group, 5 words of K and of V
  // covering this lane's 16 index bytes (start offsets are even, so the words
  // are realigned by 0 or 2 bytes -- a per-lane constant), plus the scales of
  // token `lane`.  The next tile is fetched into the same registers as soon as
  // the current tile's raw words are consumed (K realigned into registers, V
  // and the scales staged in LDS), so it is in flight during the scores,
  // softmax and PV work of the current tile.  A tile past the end of the
  // split is fetched at an offset beyond the buffer range, which the hardware
  // turns into zeros without a memory access, so every fetch is issued
  // unconditionally and the wait counts stay exact.
  // (fp16 tensors: a lane fetches its token's 32 dims, 64 aligned bytes, as 4
  // 16-byte loads; no scale.)
  // (TBQ3: a lane's 32 codes are 12 bytes at an even offset: one 16-byte
  // load at the word-aligned offset below covers them.)
  // (q8_0 K: a lane's 8 codes of each of the token's 4 blocks, 10 words;
  // q8_0 V: the lane's block -- scale and 32 codes -- in 9 words; the K
  // scales come two per lane.)
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
  // word-aligned start of this lane's code bytes of tile t, block blk
  auto code_addr = [&](bool live, int t, int blk, uint32_t bb, uint32_t per_quarter) -> uint32_t {
    if (!live) return 0xFFFF0000u;
    return ((uint32_t)(t * kTile + 16 * blk + col) * bb + 2u + per_quarter * quarter) & ~3u;
  };
  auto fetch = [&](Raw &r, int t) {
    const bool live = t < t_end;
    const uint32_t base = live ? (uint32_t)t * kTile * kBlockBytes : 0xFFFF0000u;
#pragma unroll
    for (int blk = 0; blk < kBlk; ++blk) {
      const uint32_t a = (base + (uint32_t)(16 * blk) * kBlockBytes + lane_off) & ~3u;
      if constexpr (KF == kFmtTbq4) {
        r.k4[blk] = buf_load_x4(rk, a);
        r.k1[blk] = buf_load_x1(rk, a + 16);
      } else if constexpr (KF == kFmtTbq3) {
        r.k4[blk] = buf_load_x4(rk, code_addr(live, t, blk, kBlockBytes3, 12u));
      } else if constexpr (KF == kFmtQ8) {
        // codes 8 q .. 8 q + 7 of block c start at byte 34 c + 2 + 8 q of
        // the token (token rows are 8-byte aligned): 2 bytes into a word for
        // even c, word-aligned for odd c
        const uint32_t tb =
            live ? (uint32_t)(t * kTile + 16 * blk + col) * kQ8RowBytes + 8u * quarter : 0xFFFF0000u;
        r.kq3[2 * blk] = buf_load_x3(rk, tb);
        r.kq2[2 * blk] = buf_load_x2(rk, tb + 36);
        r.kq3[2 * blk + 1] = buf_load_x3(rk, tb + 68);
        r.kq2[2 * blk + 1] = buf_load_x2(rk, tb + 104);
      } else {
        const uint32_t f = live ? ((uint32_t)(t * kTile + 16 * blk + col) * kKBytes + 64u * quarter)
                                : 0xFFFF0000u;
#pragma unroll
        for (int c = 0; c < 4; ++c) r.k4[4 * blk + c] = buf_load_x4(rk, f + 16u * c);
      }
      if constexpr (VF == kFmtTbq4) {
        r.v4[blk] = buf_load_x4(rv, a);
        r.v1[blk] = buf_load_x1(rv, a + 16);
      } else if constexpr (VF == kFmtTbq3) {
        r.v4[blk] = buf_load_x4(rv, code_addr(live, t, blk, kBlockBytes3, 12u));
      } else if constexpr (VF == kFmtQ8) {
        const uint32_t vb =
            live ? ((uint32_t)(t * kTile + 16 * blk + col) * kQ8RowBytes + 34u * quarter) & ~3u
                 : 0xFFFF0000u;
        r.v4[2 * blk] = buf_load_x4(rv, vb);
        r.v4[2 * blk + 1] = buf_load_x4(rv, vb + 16);
        r.v1[blk] = buf_load_x1(rv, vb + 32);
      } else {
        const uint32_t f = live ? ((uint32_t)(t * kTile + 16 * blk + col) * kVBytes + 64u * quarter)
                                : 0xFFFF0000u;
#pragma unroll
        for (int c = 0; c < 4; ++c) r.v4[4 * blk + c] = buf_load_x4(rv, f + 16u * c);
      }
    }
    const uint32_t soff = lane < kTile ? base + (uint32_t)lane * kBlockBytes : 0xFFFF0000u;
    const uint32_t soff3 = lane < kTile && live ? (uint32_t)(t * kTile + lane) * kBlockBytes3 : 0xFFFF0000u;
    if constexpr (KF == kFmtTbq4) r.sk = buf_load_u16(rk, soff);
    if constexpr (KF == kFmtTbq3) r.sk = buf_load_u16(rk, soff3);
    if constexpr (VF == kFmtTbq4) r.sv = buf_load_u16(rv, soff);
    if constexpr (VF == kFmtTbq3) r.sv = buf_load_u16(rv, soff3);
    if constexpr (KF == kFmtQ8) {   // lane: token lane % 32, blocks 2 (lane / 32) + 0, 1
      const uint32_t so = live ? (uint32_t)(t * kTile + (lane & 31)) * kQ8RowBytes + 68u * (lane >> 5)
                               : 0xFFFF0000u;
      r.skq[0] = buf_load_u16(rk, so);
      r.skq[1] = buf_load_u16(rk, so + 34);
    }
  };

  // the first tile's fetch is in flight while q' is formed
  Raw r;
  fetch(r, t_begin);

  // ---------------- q' = R q * scale * log2(e) (q * scale * log2(e) for an
  // fp16 or q8_0 K cache), split into an fp16 high part and residual.  Lane
  // quarter q holds the quarter's 32 elements i of each head: dims 32 q + i,
  // or for a q8_0 K cache 32 (i/8) + 8 q + i%8, so that MFMA step c spans
  // q8_0 block c.  Lanes col and col + 8 carry the same head (the high part
  // and the residual of its operand), so they share the work: lane part p =
  // col / 8 rotates and splits elements 16 p .. 16 p + 15, and the two trade
  // the fp16 words each needs from the other at the end.
  half8 qop[4];
  float qs_inv;
  {
    const int part = lo_part ? 1 : 0;
    const bool live = head < G;
    // a lane past the group reads head 0's row (in bounds) and is zeroed below
    const QT *qp = (const QT *)a.q +
                   ((size_t)b * a.n_q_heads + (size_t)g * G + (live ? head : 0)) * kHeadDim;
    float qv[16];
    if constexpr (KF == kFmtQ8) {
      load_q8<QT>(qp + 64 * part + 8 * quarter, qv);
      load_q8<QT>(qp + 64 * part + 32 + 8 * quarter, qv + 8);
    } else {
      load_q8<QT>(qp + 32 * quarter + 16 * part, qv);
      load_q8<QT>(qp + 32 * quarter + 16 * part + 8, qv + 8);
    }
    if constexpr (kKRot) {
      // signs, then the 128-point butterflies: elements 1..8 apart in
      // registers, 16 apart between the two parts (lanes 8 apart), 32 and 64
      // apart across quarters (lanes 16 and 32 apart)
      const uint32_t sw = a.sign[quarter] >> (16 * part);
#pragma unroll
      for (int j = 0; j < 16; ++j) qv[j] = ((sw >> j) & 1u) ? -qv[j] : qv[j];
#pragma unroll
      for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          if ((j & h) == 0) {
            const float x = qv[j], y = qv[j + h];
            qv[j] = x + y;
            qv[j + h] = x - y;
          }
        }
      }
      const float sg = part ? -1.0f : 1.0f;   // part 0: v + v', part 1: v' - v
#pragma unroll
      for (int j = 0; j < 16; ++j) qv[j] = fmaf(sg, qv[j], lane_xor_f32<8>(qv[j], lane));
#pragma unroll
      for (int j = 0; j < 16; j += 2) butterfly_pair<16>(qv[j], qv[j + 1]);
#pragma unroll
      for (int j = 0; j < 16; j += 2) butterfly_pair<32>(qv[j], qv[j + 1]);
    }
    // one power-of-two normalisation for the whole group: max |q'| in
    // [2^13, 2^14) keeps the fp16 high part and residual inside the fp16
    // range, and 2^-ex folds into the per-token key scale.  (The maximum of
    // |v| f is the maximum of |v| times f, rounded: rounding is monotonic.)
    const float f = (kKRot ? 0.08838834764831845f : 1.0f) * a.qscale;
    float mx = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) mx = fmaxf(mx, fabsf(qv[j]));
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
    qs_inv = ldexpf(1.0f, -ex);
    const float fs = live ? ldexpf(f, ex) : 0.0f;   // f 2^ex: exact
    // operand word k of block c holds elements (8c + e0, 8c + e0 + d): TBQ4 K
    // operands hold the 4 even then the 4 odd dims of a code word (pairs 0 2,
    // 4 6, 1 3, 5 7), the other formats 8 consecutive dims
    uint32_t hw[2][4], lw[2][4];
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int e0 = KF == kFmtTbq4 ? (k < 2 ? 4 * k : 4 * (k - 2) + 1) : 2 * k;
        const int e1 = KF == kFmtTbq4 ? e0 + 2 : e0 + 1;
        const float x0 = qv[8 * cc + e0] * fs, x1 = qv[8 * cc + e1] * fs;
        hw[cc][k] = pk_f16(x0, x1);
        lw[cc][k] = pk_f16_residual(hw[cc][k], x0, x1);
      }
    }
    // part 0 (high part) takes its own high words for blocks 0-1 and the
    // partner's for blocks 2-3; part 1 (residual) the partner's residual
    // words for blocks 0-1 and its own for 2-3
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      u32x4 w0, w1;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t rh = lane_xor<8>(hw[cc][k], lane), rl = lane_xor<8>(lw[cc][k], lane);
        w0[k] = part ? rl : hw[cc][k];
        w1[k] = part ? lw[cc][k] : rh;
      }
      qop[cc] = __builtin_bit_cast(half8, w0);
      qop[2 + cc] = __builtin_bit_cast(half8, w1);
    }
  }

  // kPartial: the tile may hold slots >= n_ctx (only the last tile of the
  // context); full tiles carry no masking code at all
  auto process = [&](Raw &r, int t, auto partial_tag) {
    constexpr bool kPartial = decltype(partial_tag)::value;
    const int tok0 = t * kTile;
    // K words taken out of the fetch registers before the refill: TBQ4 code
    // words realigned (converted to fp16 operands at the MFMA), or fp16 rows
    uint32_t kw[kBlk][4];
    u32x4 kf[KF == kFmtF16 ? kBlk * 4 : 1];
    uint32_t kq[KF == kFmtQ8 ? kBlk : 1][8];
#pragma unroll
    for (int blk = 0; blk < kBlk; ++blk) {
      if constexpr (KF == kFmtTbq4) {
        const u32x4 w = r.k4[blk];
        kw[blk][0] = alignbyte(w[1], w[0], shift);
        kw[blk][1] = alignbyte(w[2], w[1], shift);
        kw[blk][2] = alignbyte(w[3], w[2], shift);
        kw[blk][3] = alignbyte(r.k1[blk], w[3], shift);
      } else if constexpr (KF == kFmtTbq3) {
        const u32x4 w = r.k4[blk];       // 96 code bits of the lane's 32 dims
        kw[blk][0] = alignbyte(w[1], w[0], shift);
        kw[blk][1] = alignbyte(w[2], w[1], shift);
        kw[blk][2] = alignbyte(w[3], w[2], shift);
      } else if constexpr (KF == kFmtQ8) {
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
      } else {
        // fp16 slots >= n_ctx may hold anything: zero them (a NaN value would
        // survive the -inf mask)
        const bool dead = kPartial && tok0 + 16 * blk + col >= n_ctx;
#pragma unroll
        for (int c = 0; c < 4; ++c) kf[4 * blk + c] = dead ? u32x4{0u, 0u, 0u, 0u} : r.k4[4 * blk + c];
      }
    }
    auto k_operand = [&](int blk, int c) -> half8 {
      if constexpr (KF == kFmtTbq4) return word_to_half8(kw[blk][c]);
      else if constexpr (KF == kFmtTbq3)
        return tbq3_chunk_to_half8(tbq3_chunk(kw[blk][0], kw[blk][1], kw[blk][2], c));
      else if constexpr (KF == kFmtQ8) return i8x8_to_half8(kq[blk][2 * c], kq[blk][2 * c + 1]);
      else return __builtin_bit_cast(half8, kf[4 * blk + c]);
    };

    __syncthreads();   // previous tile's LDS reads are done
#pragma unroll
    for (int blk = 0; blk < kBlk; ++blk) {
      if constexpr (VF == kFmtTbq4) {
        const u32x4 w = r.v4[blk];
        const u32x4 a = {alignbyte(w[1], w[0], shift), alignbyte(w[2], w[1], shift),
                         alignbyte(w[3], w[2], shift), alignbyte(r.v1[blk], w[3], shift)};
        *(u32x4 *)(vlds + (16 * blk + col) * kVRow + 16 * quarter) = a;
      } else if constexpr (VF == kFmtTbq3) {
        // the lane's 32 codes -> 32 e4m3 bytes (dims 32 quarter ..) in LDS
        const u32x4 w = r.v4[blk];
        const uint32_t w0 = alignbyte(w[1], w[0], shift), w1 = alignbyte(w[2], w[1], shift),
                       w2 = alignbyte(w[3], w[2], shift);
        uint32_t e[8];
#pragma unroll
        for (int c = 0; c < 4; ++c) tbq3_chunk_to_e4m3(tbq3_chunk(w0, w1, w2, c), e[2 * c], e[2 * c + 1]);
        uint8_t *row = vlds + (16 * blk + col) * kE4Row + 32 * quarter;
        *(u32x4 *)row = u32x4{e[0], e[1], e[2], e[3]};
        *(u32x4 *)(row + 16) = u32x4{e[4], e[5], e[6], e[7]};
      } else if constexpr (VF == kFmtQ8) {
        // block `quarter` of the token: the scale then 32 codes, from byte
        // 0 (even quarter: codes 2 bytes into the words) or byte 2 (odd
        // quarter: codes from the second word on) of the fetched words
        const u32x4 w0 = r.v4[2 * blk], w1 = r.v4[2 * blk + 1];
        const uint32_t d[9] = {w0[0], w0[1], w0[2], w0[3], w1[0], w1[1], w1[2], w1[3], r.v1[blk]};
        const bool odd = (quarter & 1) != 0;
        uint32_t cw[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) cw[j] = odd ? d[j + 1] : alignbyte(d[j + 1], d[j], 2u);
        uint8_t *row = vlds + (16 * blk + col) * kE4Row + 32 * quarter;
        *(u32x4 *)row = u32x4{cw[0], cw[1], cw[2], cw[3]};
        *(u32x4 *)(row + 16) = u32x4{cw[4], cw[5], cw[6], cw[7]};
        const uint16_t sbits = (uint16_t)(odd ? d[0] >> 16 : d[0] & 0xFFFFu);
        const bool dead = kPartial && tok0 + 16 * blk + col >= n_ctx;   // (NaN guard)
        svq[quarter * kTile + 16 * blk + col] = dead ? 0.0f : half_bits_to_float(sbits);
      } else {
        const bool dead = kPartial && tok0 + 16 * blk + col >= n_ctx;   // (as for K)
#pragma unroll
        for (int c = 0; c < 4; ++c)
          *(u32x4 *)(vlds + (16 * blk + col) * kF16Row + 64 * quarter + 16 * c) =
              dead ? u32x4{0u, 0u, 0u, 0u} : r.v4[4 * blk + c];
      }
    }
    if (lane < kTile) {
      float dk = qs_inv, dv = 1.0f;   // (q8_0: per-block scales below)
      if constexpr (KF == kFmtTbq4 || KF == kFmtTbq3) dk = half_bits_to_float(r.sk) * qs_inv;
      if constexpr (KF == kFmtQ8) dk = 1.0f;
      if constexpr (VF == kFmtTbq4 || VF == kFmtTbq3) dv = half_bits_to_float(r.sv);
      if constexpr (kPartial) {
        // slots >= n_ctx may hold anything (a NaN scale would survive p = 0)
        if (tok0 + lane >= n_ctx) dk = dv = 0.0f;
      }
      sk[lane] = dk;
      sv[lane] = dv;
    }
    // a V scale of 256 or more (or an unused slot's bits) keeps the running
    // maximum exact for this tile: P~ = p d^V must stay below the fp16 range
    bool vbig = VF == kFmtQ8;
    if constexpr (VF == kFmtTbq4 || VF == kFmtTbq3) vbig = __any(r.sv > 0x5BFFu);
    if constexpr (KF == kFmtQ8) {
      const int tk = lane & 31, c0 = 2 * (lane >> 5);
      const bool dead = kPartial && tok0 + tk >= n_ctx;
      skq[c0 * kTile + tk] = dead ? 0.0f : half_bits_to_float(r.skq[0]) * qs_inv;
      skq[(c0 + 1) * kTile + tk] = dead ? 0.0f : half_bits_to_float(r.skq[1]) * qs_inv;
    }
    fetch(r, t + 1);   // the raw words are consumed: refill with the next tile

    // ---- scores S^T[token][col] = K . q'.  The fp16 high-part (columns
    // 0-7) and residual (columns 8-15) partial sums of a head are added by a
    // 16-lane rotation, and the two 16-token blocks share the work: lanes
    // 0-7 of each row finish block 0, lanes 8-15 block 1, so every lane
    // carries 4 distinct scores (head `head`, tokens 16 * own + 4 * quarter + e).
    // (q8_0 K: step c spans block c, whose scale differs per token, so each
    // step has its own accumulator and the scales are applied in fp32.)
    float4v acc[kBlk];
    float4v acq[KF == kFmtQ8 ? kBlk : 1][4];
#pragma unroll
    for (int blk = 0; blk < kBlk; ++blk) {
      acc[blk] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if constexpr (KF == kFmtQ8)
          acq[blk][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(k_operand(blk, c), qop[c],
                                                               float4v{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        else
          acc[blk] = __builtin_amdgcn_mfma_f32_16x16x32_f16(k_operand(blk, c), qop[c], acc[blk],
                                                            0, 0, 0);
      }
    }
    __syncthreads();   // staged V rows and scales are visible
    const int own = lo_part ? 1 : 0;
    // the lane's K and V scales first, then (TBQ4 V) the tile's transposed V
    // reads: LDS reads return in order, so the scores wait for the scales
    // only and the V reads' latency passes under the softmax rather than
    // before the PV MFMAs
    const float4v kd = *(const float4v *)(sk + 16 * own + 4 * quarter);
    const float4v vd0 = *(const float4v *)(sv_rd + 4 * quarter);        // block 0
    const float4v vd1 = *(const float4v *)(sv_rd + 16 + 4 * quarter);   // block 1
    typedef __attribute__((address_space(3))) int2v lds_i2;
    int2v vtr[VF == kFmtTbq4 ? 4 : 1];
    if constexpr (VF == kFmtTbq4) {
#pragma unroll
      for (int cg = 0; cg < 4; ++cg)
        vtr[cg] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i2 *)(vlds + tr_off + 16 * cg));
    }
    if constexpr (KF == kFmtQ8) {
#pragma unroll
      for (int blk = 0; blk < kBlk; ++blk)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const float4v kd4 = *(const float4v *)(skq + c * kTile + 16 * blk + 4 * quarter);
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[blk][e] = fmaf(kd4[e], acq[blk][c][e], acc[blk][e]);
        }
    }
    float sc[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float mine = lo_part ? acc[1][e] : acc[0][e];
      const float give = lo_part ? acc[0][e] : acc[1][e];   // what the partner lane needs
      sc[e] = mine + row_ror8(give);
    }

    // t = score - m_ref with the running max updated lazily: m_ref is the
    // reference maximum (0 before the first tile), and only a tile holding a
    // score more than kLag above it -- and the first tile -- takes the
    // rescaling path, which recovers the scores as t + m_ref and moves the
    // reference to the true maximum.  In between, p = 2^t <= 2^kLag: the
    // partial state (m_ref, l, O') is exact for any reference, and P~ = p d^V
    // <= 256 * 255.875 = 65504 stays finite in fp16 (tiles with a larger V
    // scale, and q8_0 V, use lag 0).  A reference that trails the scores by
    // up to kLag spares the rescale on data whose scores drift upward.
    const float m_ref = m_run == -INFINITY ? 0.0f : m_run;
    float t4[4];
    float tmax = -INFINITY;
    {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        t4[e] = fmaf(sc[e], kd[e], -m_ref);
        tmax = fmaxf(tmax, t4[e]);
      }
    }
    if constexpr (kPartial) {
      tmax = -INFINITY;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        t4[e] += (tok0 + 16 * own + 4 * quarter + e < n_ctx) ? 0.0f : -INFINITY;
        tmax = fmaxf(tmax, t4[e]);
      }
    }
    constexpr float kLag = 8.0f;
    if (__any(tmax > (vbig ? 0.0f : kLag) || m_run == -INFINITY)) {
      float smax = tmax + m_ref;
      smax = fmaxf(smax, __shfl_xor(smax, 8, 64));
      smax = fmaxf(smax, __shfl_xor(smax, 16, 64));
      smax = fmaxf(smax, __shfl_xor(smax, 32, 64));
      const float m_new = fmaxf(m_run, smax);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
      float al[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) al[e] = __shfl(alpha, (4 * quarter + e) & 7, 64);
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) o[i][e] *= al[e];
      const float shift_t = m_ref - m_new;
#pragma unroll
      for (int e = 0; e < 4; ++e) t4[e] += shift_t;
    }

    // ---- probabilities and P~ = p d^V, carried as an fp16 value (rows 0-7
    // of the P~ operand, lanes 0-7 of each row) plus the fp16 rounding of
    // what that value leaves out (rows 8-15, the same head's row + 8): the
    // MFMA accumulates both, and the final cross-lane sum adds row h + 8 to
    // row h, so each weight carries ~22 bits.  A single fp16 would move the
    // output by up to 2^-11 of the dominant V rows when few keys carry the
    // weight.  A row needs both blocks' tokens: its own block from itself,
    // the other from the partner lane.  Lanes 8-15 compute zeros here (they
    // read the V scales from a zero block) and receive the residual words of
    // lanes 0-7.
    float psum = 0.0f;
    float p4[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      p4[e] = __builtin_amdgcn_exp2f(t4[e]);
      psum += p4[e];
    }
    l_run += psum;
    uint32_t pw[4];   // round to nearest (v_cvt_pk_f16_f32): no truncation bias
    {
      float pt[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pt[e] = p4[e] * vd0[e];                 // lanes 0-7: own block 0
        pt[4 + e] = row_ror8(p4[e]) * vd1[e];   // partner's block 1
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) pw[j] = split_f16x2(pt[2 * j], pt[2 * j + 1]);
    }
    half8 pa[kBlk / 2];
    pa[0] = __builtin_bit_cast(half8, u32x4{pw[0], pw[1], pw[2], pw[3]});
    // q8_0 V: one P~ per 32-dim block c, p times that block's scale
    half8 paq[VF == kFmtQ8 ? 4 : 1];
    if constexpr (VF == kFmtQ8) {
      float pr[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) pr[e] = row_ror8(p4[e]);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float *svc = lo_part ? svq + 4 * kTile : svq + c * kTile;
        const float4v q0 = *(const float4v *)(svc + 4 * quarter);
        const float4v q1 = *(const float4v *)(svc + 16 + 4 * quarter);
        uint32_t qw[4];   // fp16 value and residual rows, as for the other formats
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          qw[j] = split_f16x2(p4[2 * j] * q0[2 * j], p4[2 * j + 1] * q0[2 * j + 1]);
          qw[2 + j] = split_f16x2(pr[2 * j] * q1[2 * j], pr[2 * j + 1] * q1[2 * j + 1]);
        }
        paq[c] = __builtin_bit_cast(half8, u32x4{qw[0], qw[1], qw[2], qw[3]});
      }
    }

    // ---- O'^T += P~ V
    if constexpr (VF == kFmtTbq4) {
      // V read back transposed: 8 tokens x 1 byte (2 dims) per lane
      static_assert(kBlk / 2 == 1, "one 32-token P~ operand per tile");
#pragma unroll
      for (int kk = 0; kk < kBlk / 2; ++kk) {
#pragma unroll
        for (int cg = 0; cg < 4; ++cg) {
          const int2v r = vtr[cg];
          const uint32_t w0 = (uint32_t)r[0], w1 = (uint32_t)r[1];
          const half8 ve = lo_nibbles_to_half8(w0, w1);
          const half8 vo = lo_nibbles_to_half8(w0 >> 4, w1 >> 4);
          o[2 * cg] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa[kk], ve, o[2 * cg], 0, 0, 0);
          o[2 * cg + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa[kk], vo, o[2 * cg + 1], 0, 0, 0);
        }
      }
    } else if constexpr (VF == kFmtQ8) {
      // q8_0 V staged as int8 codes: one byte-transposed read per 16 dims
      // (dims 16 db .. lie in block db / 2)
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        typedef __attribute__((address_space(3))) int2v lds_i2;
        const int2v rr = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i2 *)(vlds + tr8_3_off + 16 * db));
        o[db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
            paq[db >> 1], i8x8_to_half8((uint32_t)rr[0], (uint32_t)rr[1]), o[db], 0, 0, 0);
      }
    } else if constexpr (VF == kFmtTbq3) {
      // TBQ3 V staged as e4m3 bytes: one byte-transposed read per 16 dims
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        typedef __attribute__((address_space(3))) int2v lds_i2;
        const int2v rr = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i2 *)(vlds + tr8_3_off + 16 * db));
        o[db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
            pa[0], e4m3x8_to_half8((uint32_t)rr[0], (uint32_t)rr[1]), o[db], 0, 0, 0);
      }
    } else {
      // fp16 V: two 16-bit transposed reads give a lane 8 tokens of one dim
      // (dim 16 db + col); source lanes point at token 4 quarter + col / 4
      // (+ 16 for the second read) and dims 4 (col % 4) .. + 3 of the block
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        typedef __attribute__((address_space(3))) short4v lds_s4;
        const short4v r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4 *)(vlds + tr16_off + 32 * db));
        const short4v r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s4 *)(vlds + tr16_off + 16 * kF16Row + 32 * db));
        const short8v vv = {r0[0], r0[1], r0[2], r0[3], r1[0], r1[1], r1[2], r1[3]};
        o[db] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa[0], __builtin_bit_cast(half8, vv), o[db],
                                                       0, 0, 0);
      }
    }
  };

  const int t_full = min(t_end, n_ctx / kTile);   // tiles below t_full are full
  int t = t_begin;
  for (; t < t_full; ++t) process(r, t, std::false_type{});
  for (; t < t_end; ++t) process(r, t, std::true_type{});

  // ---------------- partial state of this split
  l_run += lane_xor_f32<8>(l_run, lane);
  l_run += lane_xor_f32<16>(l_run, lane);
  l_run += lane_xor_f32<32>(l_run, lane);

  const int P = a.n_splits;
  float *wsb = a.ws + ((size_t)b * a.n_q_heads + (size_t)g * G) * P * 130 + (size_t)split * 130;
  if (lane < G) {
    wsb[(size_t)lane * P * 130 + 0] = m_run;
    wsb[(size_t)lane * P * 130 + 1] = l_run;
  }
  // O'^T rows h and h + 8 (lanes l and l + 32) add up to head h's output.
  // Accumulators pair up (o[2k], o[2k+1]): one swap of the halves leaves
  // each lane of the lower half a value of o[2k] and its partner, and each
  // lane of the upper half a value of o[2k+1] and its partner, so one add
  // forms both registers' sums and all 64 lanes store: lanes 0-31 the dims
  // of o[2k], lanes 32-63 those of o[2k+1], for heads 4 (quarter % 2) + e.
  const int hsel = quarter >> 1;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(o[2 * k][e]),
                                                       __float_as_uint(o[2 * k + 1][e]), false, false);
      const float s = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
      const int r = 4 * (quarter & 1) + e;   // query head within the group
      if (r < G) {
        // TBQ4 V: o[2k] holds dims 32 k + 2 col, o[2k+1] the odd dims after
        // them; the other formats: o[db] holds dims 16 db + col
        const int d = VF == kFmtTbq4 ? 32 * k + 2 * col + hsel : 16 * (2 * k + hsel) + col;
        wsb[(size_t)r * P * 130 + 2 + d] = s;
      }
    }
  }
}

// Merge: o = R^T (sum_p 2^(m_p - M) o'_p / sum_p 2^(m_p - M) l_p), one
// workgroup of NW wavefronts per (sequence, query head), in one pass over the
// partials.  Wavefront w takes splits w, w + NW, ... in chunks of
// kMergeChunk (lane holds dims lane and lane + 64), all loads of a chunk in
// flight together, combined under a running maximum; the wavefronts' sums
// meet in LDS, rescaled to the common maximum, and wavefront 0 normalises,
// applies the inverse rotation and stores.  Empty splits carry m = -inf and
// weigh 0.  NW grows with the split count (kMergeChunk NW splits per round)
// so that up to 272 splits are read in one round of loads; 17 per wavefront
// let a decode step's extra partial state (the new token's, after 64, 128 or
// 256 splits) in without a larger workgroup or a second round.
constexpr int kMergeChunk = 17;   // partial states per wavefront and round of loads

template <typename OT, int NW>
__global__ __launch_bounds__(64 * NW) void decode_merge_kernel(DecodeArgs a) {
  __shared__ float red[NW][130];   // o'[128], l, m per wavefront
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = blockIdx.x, b = blockIdx.y;
  const int P = a.n_splits;
  const float *base = a.ws + ((size_t)b * a.n_q_heads + h) * P * 130;

  float M = -INFINITY, L = 0.0f, o0 = 0.0f, o1 = 0.0f;
  for (int p0 = wave; p0 < P; p0 += kMergeChunk * NW) {
    float mp[kMergeChunk], lp[kMergeChunk], x0[kMergeChunk], x1[kMergeChunk];
#pragma unroll
    for (int u = 0; u < kMergeChunk; ++u) {
      // splits past P reread split p0 (valid: p0 < P) and weigh 0, so that
      // the chunk's loads issue together without branches
      const int p = p0 + NW * u;
      const float *bp = base + (size_t)(p < P ? p : p0) * 130;
      mp[u] = bp[0];
      lp[u] = bp[1];
      x0[u] = bp[2 + lane];
      x1[u] = bp[66 + lane];
    }
#pragma unroll
    for (int u = 0; u < kMergeChunk; ++u)
      if (p0 + NW * u >= P) mp[u] = -INFINITY;
    float cm = M;
#pragma unroll
    for (int u = 0; u < kMergeChunk; ++u) cm = fmaxf(cm, mp[u]);
    if (cm == -INFINITY) continue;   // only empty splits so far (wavefront-uniform)
    const float al = __builtin_amdgcn_exp2f(M - cm);   // 0 while M is -inf
    L *= al;
    o0 *= al;
    o1 *= al;
#pragma unroll
    for (int u = 0; u < kMergeChunk; ++u) {
      const float wt = __builtin_amdgcn_exp2f(mp[u] - cm);
      L = fmaf(wt, lp[u], L);
      o0 = fmaf(wt, x0[u], o0);
      o1 = fmaf(wt, x1[u], o1);
    }
    M = cm;
  }
  red[wave][lane] = o0;
  red[wave][64 + lane] = o1;
  if (lane == 0) {
    red[wave][128] = L;
    red[wave][129] = M;
  }
  __syncthreads();
  if (wave != 0) return;
  float Mx = red[0][129];
#pragma unroll
  for (int w = 1; w < NW; ++w) Mx = fmaxf(Mx, red[w][129]);
  o0 = o1 = L = 0.0f;
  if (Mx != -INFINITY) {   // every split empty (a zero-length sequence): output 0
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float sw = __builtin_amdgcn_exp2f(red[w][129] - Mx);
      o0 = fmaf(sw, red[w][lane], o0);
      o1 = fmaf(sw, red[w][64 + lane], o1);
      L = fmaf(sw, red[w][128], L);
    }
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  o0 *= inv;
  o1 *= inv;
  OT *dst = (OT *)a.out + ((size_t)b * a.n_q_heads + h) * kHeadDim;
  if (!a.rotate_out) {   // an fp16 V cache is not rotated
    dst[lane] = (OT)o0;
    dst[lane + 64] = (OT)o1;
    return;
  }
  // o = s * (H o') / sqrt(128); the butterflies across lanes use DPP and
  // permlane exchanges (no LDS round trip on this serial chain)
  auto level = [&](auto hc) {
    constexpr int hh = decltype(hc)::value;
    const float p0 = lane_xor_f32<hh>(o0, lane), p1 = lane_xor_f32<hh>(o1, lane);
    const bool upper = (lane & hh) != 0;
    o0 = upper ? (p0 - o0) : (o0 + p0);
    o1 = upper ? (p1 - o1) : (o1 + p1);
  };
  level(std::integral_constant<int, 1>{});
  level(std::integral_constant<int, 2>{});
  level(std::integral_constant<int, 4>{});
  level(std::integral_constant<int, 8>{});
  level(std::integral_constant<int, 16>{});
  level(std::integral_constant<int, 32>{});
  {
    const float x = o0, y = o1;
    o0 = x + y;
    o1 = x - y;
  }
  const float r = 0.08838834764831845f;
  const bool n0 = (a.sign[lane >> 5] >> (lane & 31)) & 1u;
  const bool n1 = (a.sign[2 + (lane >> 5)] >> (lane & 31)) & 1u;
  o0 = n0 ? -o0 * r : o0 * r;
  o1 = n1 ? -o1 * r : o1 * r;
  dst[lane] = (OT)o0;
  dst[lane + 64] = (OT)o1;
}

// ---------------------------------------------------------------------------
// Scratch of the no-allocation decode entry point (for callers that cannot
// allocate device memory): the split-K partial states of a call live in this
// file-scope device array, one copy per device, held until the process ends.
// In host code `scratch` is only a host-side stand-in for the symbol: its
// device address is looked up per device with hipGetSymbolAddress (with that
// device current) and that address is what the kernels receive.  Every call on
// a device shares the device's copy, so calls that overlap on one device race.
// ---------------------------------------------------------------------------
static __device__ __align__(256) uint8_t scratch[kDecodeScratchBytes];

hipError_t decode_scratch(hipStream_t stream, void **ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void *addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    int cur = 0;
    if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_decode_partial(const DecodeArgs &a, int batch, int q_dtype, hipStream_t stream,
                                 hipEvent_t start, hipEvent_t stop) {
  // (the decode step: a 1-D grid, streaming splits first, new-token
  // wavefronts last)
  // (n_splits - 1 streaming splits + 2 new-token wavefronts per row)
  const int64_t n_wg = (int64_t)(a.n_splits + 1) * a.n_kv_heads * batch;
  if (a.step && n_wg > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 grid = a.step ? dim3((unsigned)n_wg, 1, 1) : dim3(a.n_splits, a.n_kv_heads, batch);
  // (q dtype, K format, V format) -> kernel instance
#define TBQ4_DEC(QT, KF, VF) reinterpret_cast<const void *>(&decode_split_kernel<QT, KF, VF>)
#define TBQ4_DEC_K(QT, KF) {TBQ4_DEC(QT, KF, 0), TBQ4_DEC(QT, KF, 1), TBQ4_DEC(QT, KF, 2), TBQ4_DEC(QT, KF, 3)}
  // q dtype: fp32, fp16, bf16 (16-bit patterns)
  static const void *const kernels[3][kNumFormats][kNumFormats] = {
      {TBQ4_DEC_K(float, 0), TBQ4_DEC_K(float, 1), TBQ4_DEC_K(float, 2), TBQ4_DEC_K(float, 3)},
      {TBQ4_DEC_K(_Float16, 0), TBQ4_DEC_K(_Float16, 1), TBQ4_DEC_K(_Float16, 2),
       TBQ4_DEC_K(_Float16, 3)},
      {TBQ4_DEC_K(uint16_t, 0), TBQ4_DEC_K(uint16_t, 1), TBQ4_DEC_K(uint16_t, 2),
       TBQ4_DEC_K(uint16_t, 3)}};
#undef TBQ4_DEC_K
#undef TBQ4_DEC
  if (a.k_fmt < 0 || a.k_fmt >= kNumFormats || a.v_fmt < 0 || a.v_fmt >= kNumFormats)
    return hipErrorInvalidValue;
  if (q_dtype < 0 || q_dtype > 2) return hipErrorInvalidValue;
  const void *fn = kernels[q_dtype][a.k_fmt][a.v_fmt];
  DecodeArgs arg = a;
  void *params[] = {&arg};
  if (start || stop)
    return hipExtLaunchKernel(fn, grid, dim3(64), params, 0, stream, start, stop, 0);
  return hipLaunchKernel(fn, grid, dim3(64), params, 0, stream);
}

hipError_t launch_decode_merge(const DecodeArgs &a, int batch, int out_dtype, hipStream_t stream) {
  dim3 grid(a.n_q_heads, batch);
  // wavefronts per workgroup: all splits in one round of 16 per wavefront
  const int nw = a.n_splits <= 4 * kMergeChunk ? 4 : a.n_splits <= 8 * kMergeChunk ? 8 : 16;
  static const void *const kernels[2][3] = {
      {reinterpret_cast<const void *>(&decode_merge_kernel<float, 4>),
       reinterpret_cast<const void *>(&decode_merge_kernel<float, 8>),
       reinterpret_cast<const void *>(&decode_merge_kernel<float, 16>)},
      {reinterpret_cast<const void *>(&decode_merge_kernel<_Float16, 4>),
       reinterpret_cast<const void *>(&decode_merge_kernel<_Float16, 8>),
       reinterpret_cast<const void *>(&decode_merge_kernel<_Float16, 16>)}};
  const void *fn = kernels[out_dtype == 0 ? 0 : 1][nw == 4 ? 0 : nw == 8 ? 1 : 2];
  DecodeArgs arg = a;
  void *params[] = {&arg};
  return hipLaunchKernel(fn, grid, dim3(64 * nw), params, 0, stream);
}

}  // namespace tbq4
