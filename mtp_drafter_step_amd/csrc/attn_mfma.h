// One 16-key batch of the matrix-core single-query attention, shared by the per-launch attention kernel
// (k_attention.hip) and the persistent drafter kernel (k_team.hip).
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

// One batch of 16 keys for one wave of k_attn_mfma: scores of the keys in ka against the G heads, online softmax
// update, and P V into acc. PF: the next batch's key loads (into kn) are issued first, to arrive during this batch's
// arithmetic, and become ka at the end; the last batch of a wave issues none, since copying them into ka would wait
// for loads nobody uses. The two forms are separate instances, so that the loads of the first are unconditional
// (loads under a run-time branch make every later wait count assume the branch was not taken).
// STAGED: the batch's 16 key rows already sit in `tile` (rows of LROW = 264 elements) and ka was read from there, so
// the V tile is not written again.
template <int G, bool PF, bool STAGED = false>
__device__ __forceinline__ void mfma_batch(int t0, int k1, const uint16_t* Kb, const uint16_t* Vb, int cap,
                                           bool same_v, float scale_log2, uint16_t* tile,
                                           const uint16_t (*qop)[2][G][4][8], uint4 (&ka)[8], uint4 (&kn)[8],
                                           f32x4 (&acc)[16], float& mrun, float& lrun) {
  constexpr int HD = 256, KSTEPS = 8, TILES = 16, LROW = HD + 8, S = 64;
  constexpr int GQ = (G + 3) / 4;
  const int lane = lane_id(), hq = lane & 15, kq = lane >> 4;
  const int hsel = hq < G ? hq : 0;
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
  // scores S[key 4kq + r][head hq]
  f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < KSTEPS; ++c) {
    const bf16x8 a = __builtin_bit_cast(bf16x8, ka[c]);
    uint4 hi = *reinterpret_cast<const uint4*>(&qop[c][0][hsel][kq][0]);
    uint4 lo = *reinterpret_cast<const uint4*>(&qop[c][1][hsel][kq][0]);
    if (hq >= G) hi = lo = make_uint4(0u, 0u, 0u, 0u);
    sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, hi), sacc, 0, 0, 0);
    sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, lo), sacc, 0, 0, 0);
  }
  float sv[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) sv[r] = (4 * kq + r < nk && hq < G) ? sacc[r] * scale_log2 : -INFINITY;
  float mt = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
  mt = fmaxf(mt, xr_partner<16>(mt));
  mt = fmaxf(mt, xr_partner<32>(mt));
  const float mn = fmaxf(mrun, mt);
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
  uint32_t ph2[2], pl2[2];
  split_bf16x2(pv[0], pv[1], ph2[0], pl2[0]);
  split_bf16x2(pv[2], pv[3], ph2[1], pl2[1]);
  const i16x4 phi = __builtin_bit_cast(i16x4, make_uint2(ph2[0], ph2[1]));
  const i16x4 plo = __builtin_bit_cast(i16x4, make_uint2(pl2[0], pl2[1]));
  // rescale the accumulators only when some head's maximum moved (alpha is exactly 1 otherwise): D rows are heads
  // 4kq + r, whose alpha lives in lane 4kq + r (rows of heads >= G are padding)
  if (__any(alpha != 1.0f)) {
    float al[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      al[r] = readlane_f(alpha, r);
      if constexpr (GQ > 1) al[r] = (kq == 1) ? readlane_f(alpha, 4 + r) : al[r];
    }
#pragma unroll
    for (int t = 0; t < TILES; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[t][r] *= al[r];
  }
  // V operand: keys 4 kq + r of dim 16 t + hq, one transposing read of the 4 x 16 block at row 4 kq
  const uint16_t* vrow = tile + (4 * kq + (hq >> 2)) * LROW + 4 * (hq & 3);
#pragma unroll
  for (int t = 0; t < TILES; ++t) {
    const i16x4 vb = lds_read_tr16(vrow + 16 * t);
    f32x4 a = acc[t];
    a = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(phi, vb, a, 0, 0, 0);
    a = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(plo, vb, a, 0, 0, 0);
    acc[t] = a;
  }
  if constexpr (PF) {
#pragma unroll
    for (int c = 0; c < KSTEPS; ++c) ka[c] = kn[c];
  }
}

}  // namespace
}  // namespace mtpd

#endif  // MTPD_ATTN_MFMA_H
