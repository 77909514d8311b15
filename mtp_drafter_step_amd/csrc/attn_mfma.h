// One 16-key batch of the matrix-core single-query attention, shared by the per-launch attention kernel
// (k_attention.hip) and the persistent drafter kernel (k_team.hip), and the persistent kernel's variant for keys
// held in LDS that splits the output dims over the waves (mfma_tiles2_dims).
//
// Pages cited (by title; sections as headed on each page):
//   [MTP doc]    "Gemma 4 Multi-Token Prediction (MTP) drafter" (llama.cpp fork, gemma4-assistant.md)
//   [Inventory]  "Gemma 4 Assistant (MTP drafter) - tensor inventory (Stage 0)"
// Single-query attention over the target's shared cache: [MTP doc] "What it is"; V taken from K: [Inventory]
// "Notes for llama.cpp port" 2.
#ifndef MTPD_ATTN_MFMA_H
#define MTPD_ATTN_MFMA_H

#include "device.h"

namespace mtpd {
namespace {

// One batch of 16 keys for one wave of k_attn_mfma: scores of the keys in ka against the G <= 8 heads, online
// softmax update, and P V into acc (hi and lo parts of P in separate rows until attn_fold_rows). PF: the next batch's key loads (into kn) are issued first, to arrive during this batch's
// arithmetic, and become ka at the end; the last batch of a wave issues none, since copying them into ka would wait
// for loads nobody uses. The two forms are separate instances, so that the loads of the first are unconditional
// (loads under a run-time branch make every later wait count assume the branch was not taken).
// STAGED: the batch's 16 key rows already sit in `tile` (rows of LROW = 264 elements) and ka was read from there, so
// the V tile is not written again.
template <int G, bool PF, bool STAGED = false>
__device__ __forceinline__ void mfma_batch(int t0, int k1, const uint16_t* Kb, const uint16_t* Vb, int cap,
                                           bool same_v, float scale_log2, uint16_t* tile,
                                           const uint16_t (*qop)[2][8][4][8], uint4 (&ka)[8], uint4 (&kn)[8],
                                           f32x4 (&acc)[16], float& mrun, float& lrun, int h0 = 0, int h1 = G) {
  constexpr int HD = 256, KSTEPS = 8, TILES = 16, LROW = HD + 8, S = 64;
  constexpr int GQ = (G + 3) / 4;
  const int lane = lane_id(), hq = lane & 15, kq = lane >> 4;
  const int tb = t0;
  if constexpr (PF) {
    const uint16_t* r = Kb + (size_t)slot_of(min(t0 + S + hq, k1 - 1), cap) * HD;
#pragma unroll
    for (int c = 0; c < KSTEPS; ++c) kn[c] = *reinterpret_cast<const uint4*>(r + 32 * c);
  }
  const int nk = min(16, k1 - tb);
  // V tile into this wave's LDS (row = key hq, dims 32c + 8kq .. +8)
  if constexpr (STAGED) {
  } else if (same_v) {
#pragma unroll
    for (int c = 0; c < KSTEPS; ++c) *reinterpret_cast<uint4*>(tile + hq * LROW + 32 * c + 8 * kq) = ka[c];
  } else {
    const uint16_t* r = Vb + (size_t)slot_of(min(tb + hq, k1 - 1), cap) * HD;
    uint4 vv[KSTEPS];
#pragma unroll
    for (int c = 0; c < KSTEPS; ++c) vv[c] = *reinterpret_cast<const uint4*>(r + 32 * c);
#pragma unroll
    for (int c = 0; c < KSTEPS; ++c) *reinterpret_cast<uint4*>(tile + hq * LROW + 32 * c + 8 * kq) = vv[c];
  }
  // scores: column n < G of the tile takes q_hi of head n, column 8 + n takes q_lo of head n (qop holds zeros for
  // the other columns), so one product covers both terms; lane hq < G adds its column 8 + hq partner, 8 lanes away
  // in its row of 16. All eight B operands are read before the products, so the reads overlap.
  f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
  {
    uint4 qb[KSTEPS];
#pragma unroll
    for (int c = 0; c < KSTEPS; ++c) qb[c] = *reinterpret_cast<const uint4*>(&qop[c][hq >> 3][hq & 7][kq][0]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int c = 0; c < KSTEPS; ++c)
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ka[c]), __builtin_bit_cast(bf16x8, qb[c]),
                                                     sacc, 0, 0, 0);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) sacc[r] += xr_partner<8>(sacc[r]);
  float sv[4];
#pragma unroll
  // columns h0 .. h1 - 1 only: the query heads that read this batch's kv head (the others see no key here)
  for (int r = 0; r < 4; ++r) sv[r] = (4 * kq + r < nk && hq >= h0 && hq < h1) ? sacc[r] * scale_log2 : -INFINITY;
  float mt = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
  mt = fmaxf(mt, xr_partner<16>(mt));
  mt = fmaxf(mt, xr_partner<32>(mt));
  // the reference maximum moves only when a score exceeds it by more than 2^8: below that the weights stay under
  // 256, far inside fp32 and exact in the bf16 hi + lo split, and most batches skip the rescale
  const float mn = (mt > mrun + 8.0f) ? mt : mrun;
  // 2^x on the hardware instruction: weights below 2^-126 flush to zero, far below what a weight contributes
  const float alpha = (mrun == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mrun - mn);
  float pv[4], ps = 0.f;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    pv[r] = (sv[r] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(sv[r] - mn);
    ps += pv[r];
  }
  ps += xr_partner<16>(ps);
  ps += xr_partner<32>(ps);
  lrun = lrun * alpha + ps;
  mrun = mn;
  // P operand: row h < G holds the bf16 hi part of head h's weights, row 8 + h the lo part (taken from lane h, 8
  // lanes away); the output rows 8 + h therefore collect the lo products, folded in by attn_fold_rows
  uint32_t ph2[2], pl2[2];
  split_bf16x2(pv[0], pv[1], ph2[0], pl2[0]);
  split_bf16x2(pv[2], pv[3], ph2[1], pl2[1]);
  uint32_t pa[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const uint32_t lo8 = __float_as_uint(xr_partner<8>(__uint_as_float(pl2[i])));
    pa[i] = (hq < 8) ? ph2[i] : lo8;
  }
  const i16x4 pop = __builtin_bit_cast(i16x4, make_uint2(pa[0], pa[1]));
  // rescale the accumulators only when some head's maximum moved (alpha is exactly 1 otherwise): D row 4kq + r
  // belongs to head (4kq + r) mod 8, whose alpha lives in that lane (rows of no head are zero)
  if (__any(hq < G && alpha != 1.0f)) {
    float al[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      al[r] = readlane_f(alpha, r);
      if constexpr (GQ > 1) al[r] = (kq & 1) ? readlane_f(alpha, 4 + r) : al[r];
    }
#pragma unroll
    for (int t = 0; t < TILES; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[t][r] *= al[r];
  }
  // V operand: keys 4 kq + r of dim 16 t + hq, one transposing read of the 4 x 16 block at row 4 kq
  const uint16_t* vrow = tile + (4 * kq + (hq >> 2)) * LROW + 4 * (hq & 3);
  i16x4 vb[TILES];
#pragma unroll
  for (int t = 0; t < TILES; ++t) vb[t] = lds_read_tr16(vrow + 16 * t);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int t = 0; t < TILES; ++t) acc[t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pop, vb[t], acc[t], 0, 0, 0);
  if constexpr (PF) {
#pragma unroll
    for (int c = 0; c < KSTEPS; ++c) ka[c] = kn[c];
  }
}

// Two 16-key tiles (32 keys from tb) of a split whose keys sit in LDS (`tile`: the first tile's row, rows of 264
// elements; ka[i] holds tile i's rows as read from there), scored against the 4 heads whose q operand is in qop, with
// P V taken for dims 64 dq .. 64 dq + 63 only (acc[t] covers dims 64 dq + 16 t + hq). The two tiles' score products
// are independent chains, one softmax update covers all 32 keys, and P V runs as v_mfma_f32_16x16x32_bf16 over the
// 32 keys. Every wave of a block runs the same scores and softmax on the same keys, so the waves' (max, sum) states
// are identical and a wave's 64 dims need no combine with the other waves. Row layout of acc as in mfma_batch: rows
// 0 .. 3 the hi products of heads 0 .. 3, rows 8 .. 11 their lo products. Only heads h0 .. h1 - 1 read these keys
// (the query heads of the tile's kv head); the others get no weight from them.
__device__ __forceinline__ void mfma_tiles2_dims(int tb, int k1, float scale_log2, const uint16_t* tile,
                                                 const uint16_t (*qop)[2][8][4][8], const uint4 (&ka)[2][8], int dq,
                                                 f32x4 (&acc)[4], float& mrun, float& lrun, int h0 = 0, int h1 = 4) {
  constexpr int KSTEPS = 8, LROW = 264;
  const int lane = lane_id(), hq = lane & 15, kq = lane >> 4;
  f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
  {
    uint4 qb[KSTEPS];
#pragma unroll
    for (int c = 0; c < KSTEPS; ++c) qb[c] = *reinterpret_cast<const uint4*>(&qop[c][hq >> 3][hq & 7][kq][0]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int c = 0; c < KSTEPS; ++c)
#pragma unroll
      for (int i = 0; i < 2; ++i)
        sacc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ka[i][c]),
                                                          __builtin_bit_cast(bf16x8, qb[c]), sacc[i], 0, 0, 0);
  }
  // scores of keys tb + 16 i + 4 kq + r in sv[4 i + r] (column hq: head hq once the lo column is added)
  float sv[8];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float s = sacc[i][r] + xr_partner<8>(sacc[i][r]);
      sv[4 * i + r] = (tb + 16 * i + 4 * kq + r < k1 && hq >= h0 && hq < h1) ? s * scale_log2 : -INFINITY;
    }
  float mt = sv[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) mt = fmaxf(mt, sv[i]);
  mt = fmaxf(mt, xr_partner<16>(mt));
  mt = fmaxf(mt, xr_partner<32>(mt));
  // lazy maximum as in mfma_batch: it moves only when a score exceeds it by more than 2^8
  const float mn = (mt > mrun + 8.0f) ? mt : mrun;
  const float alpha = (mrun == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mrun - mn);
  float pv[8], ps = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    pv[i] = (sv[i] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(sv[i] - mn);
    ps += pv[i];
  }
  ps += xr_partner<16>(ps);
  ps += xr_partner<32>(ps);
  lrun = lrun * alpha + ps;
  mrun = mn;
  // P as the A operand over the 32 keys: lane (hq, kq) supplies k = 8 kq + i, standing for key 4 kq + i (i < 4) and
  // key 16 + 4 kq + i - 4; row hq < 8 the hi parts of head hq, row 8 + h the lo parts of head h (from lane h)
  uint32_t ph[4], pl[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) split_bf16x2(pv[2 * i], pv[2 * i + 1], ph[i], pl[i]);
  uint32_t pa[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo8 = __float_as_uint(xr_partner<8>(__uint_as_float(pl[i])));
    pa[i] = (hq < 8) ? ph[i] : lo8;
  }
  const bf16x8 pop = __builtin_bit_cast(bf16x8, make_uint4(pa[0], pa[1], pa[2], pa[3]));
  if (__any(hq < 4 && alpha != 1.0f)) {
    float al[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) al[r] = readlane_f(alpha, r);
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[t][r] *= al[r];
  }
  // V operand in the same key order: two transposing reads, at key rows 4 kq and 16 + 4 kq
  const uint16_t* vrow = tile + (4 * kq + (hq >> 2)) * LROW + 4 * (hq & 3) + 64 * dq;
  bf16x8 vb[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const i16x4 v0 = lds_read_tr16(vrow + 16 * t);
    const i16x4 v1 = lds_read_tr16(vrow + 16 * LROW + 16 * t);
    vb[t] = __builtin_bit_cast(bf16x8, (i16x8){v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]});
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int t = 0; t < 4; ++t) acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pop, vb[t], acc[t], 0, 0, 0);
}

// After the last batch: output rows 8 .. 15 hold the lo-part products of the heads in rows 0 .. 7; rows 4kq + r of
// lane (hq, kq) and (hq, kq ^ 2) are 8 rows apart, so one exchange over lanes 32 apart leaves every head's full
// accumulator in the lanes of kq = 0, 1 (and a copy in kq = 2, 3).
__device__ __forceinline__ void attn_fold_rows(f32x4 (&acc)[16]) {
#pragma unroll
  for (int t = 0; t < 16; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[t][r] += xr_partner<32>(acc[t][r]);
}

}  // namespace
}  // namespace mtpd

#endif  // MTPD_ATTN_MFMA_H
