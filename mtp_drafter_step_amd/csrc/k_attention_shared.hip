// Multi-query attention over one cache shared by every row of the batch (rows of one sequence scored together).
//
// Pages cited (by title; sections as headed on each page):
//   [MTP doc]    "Gemma 4 Multi-Token Prediction (MTP) drafter" (llama.cpp fork, gemma4-assistant.md)
//   [Guide]      "Gemma 4 Assistant 使用指南：用 MTP 投机解码与 KV Sharing 加速 Gemma 4 推理" (gitcode blog)
//   [Inventory]  "Gemma 4 Assistant (MTP drafter) - tensor inventory (Stage 0)"
//
// The attention itself is the per-row one ([MTP doc] "What it is": Q-only attention on the target's last-layer
// K/V; [Guide] section 2(4); [Inventory] "Notes for llama.cpp port" 2: V taken from K): each row's queries over its
// own key window. Only the schedule differs: the rows meet each key once.
#include "device.h"

namespace mtpd {
namespace {

// ------------------------------------------------------------------------------------------------------------
// Multi-query matrix-core attention over a cache shared by the batch's rows (rows of one sequence scored together):
// every row reads the same keys, so the query rows meet each key tile once. A block holds 128 queries (8 waves x 16
// queries: 16 / G rows x the G query heads of kv head blockIdx.z) and one key range: split blockIdx.x of the union
// [u0, u1) of the rows' windows. Key tiles of 128 rows are staged row-major in LDS for all waves (double-buffered,
// one barrier per tile): the scores read key rows, the P.V operand reads the same tile column-wise with transposing
// LDS reads. Per wave and 32-key batch (two 16-key score tiles):
//   S^T[16 keys][16 queries] = K_tile . Q^T with v_mfma_f32_16x16x32_bf16, the keys as A rows from LDS and the
//     queries as B columns held in registers as bf16 hi + lo (q after q_norm and rotation, fp32-level accuracy);
//   online softmax per query (lane column), each key masked by the query row's own window;
//   O[16 queries][256] += P . V with v_mfma_f32_16x16x16_bf16, P split hi + lo, V read from the LDS tile.
// Each wave's queries are its own, so the outputs need no combine: (max, sum) and the unnormalised sums go to the
// split partials that the o_proj kernel merges (or, with one split, straight to o).
// grid (nsplit, ceil(B / (128 / G)), n_kv), 512 threads.
// LDS row of a staged key: 544 B (256 elements and 32 B of padding), with the 16-byte columns of rows 8 .. 15 of
// every 16 swapped in pairs (column c at c ^ 1). With 64 four-byte banks a row starts two 16-byte bank groups after
// the previous one, so the 16 rows of a key read (one column each), the 8 rows of half a transposing V read (one
// column pair each) and the 16 columns of a row store all fall in distinct banks.
constexpr int kMqRow = 256 + 16;
__device__ __forceinline__ int mq_swz(int row) { return (row >> 3) & 1; }

// Part x of a key tile starting at key tb (keys 32 x .. +32, clamped into the range ending at k1): thread tid
// loads dims 8 (tid % 32) .. +8 of keys 32 x + tid / 32 and 32 x + 16 + tid / 32, so a wave reads two whole keys
// per load; mq_store_part writes them to the same places of a row-major LDS tile.
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void mq_load_part(const uint16_t* Kb, int cap, int k1, int tb, int x, int tid,
                                             u32x4 (&r)[2]) {
  const int kr = tid >> 5, dc = tid & 31;
#pragma unroll
  for (int j = 0; j < 2; ++j)
    r[j] = *reinterpret_cast<const u32x4*>(Kb + (size_t)slot_of(min(tb + 32 * x + 16 * j + kr, k1 - 1), cap) * 256 +
                                           8 * dc);
}
__device__ __forceinline__ void mq_store_part(uint16_t* tile, int x, int tid, const u32x4 (&r)[2]) {
  const int kr = tid >> 5, dc = tid & 31;
#pragma unroll
  for (int j = 0; j < 2; ++j)
    *reinterpret_cast<u32x4*>(tile + (32 * x + 16 * j + kr) * kMqRow + 8 * (dc ^ mq_swz(kr))) = r[j];
}

template <int G>
__global__ __launch_bounds__(512, 1) void k_attn_mq(int B, int nh, int nkv, const float* __restrict__ q,
                                                    const uint16_t* __restrict__ qnorm, float eps,
                                                    const float* __restrict__ rope, int type,
                                                    const uint16_t* __restrict__ K, int cap, RowWindows win,
                                                    int nsplit, int u0, int u1, float scale_log2,
                                                    float* __restrict__ pacc, float* __restrict__ pml,
                                                    float* __restrict__ o) {
  constexpr int HD = 256, KSTEPS = HD / 32, TILES = HD / 16, NW = 8, KT = 128, LROW = kMqRow, half = HD / 2;
  constexpr int RPW = 16 / G, RPB = NW * RPW;  // rows per wave, per block
  static_assert(G == 1 || G == 2 || G == 4 || G == 8, "16 queries per wave are whole rows");
  __shared__ __attribute__((aligned(16))) uint16_t kt[2][KT][LROW];
  const int sp = blockIdx.x, g = blockIdx.z;
  const int wave = wave_id(), lane = lane_id(), tid = threadIdx.x;
  const int hq = lane & 15, kq = lane >> 4;
  const int rbase = blockIdx.y * RPB + wave * RPW;  // the wave's first row
  // the lane's query: row rbase + hq / G, head g G + hq % G; rows past B repeat the last row and store nothing
  const int rq = min(rbase + hq / G, B - 1);
  const bool qlive = rbase + hq / G < B;
  const int head = g * G + hq % G;
  int wst = 0, wen = 0;  // the query row's window (virtual indices), from wave-uniform reads of the row table
  {
    // all of the wave's table reads first, so that they go out together instead of one after another
    int st[RPW], ct[RPW];
#pragma unroll
    for (int j = 0; j < RPW; ++j) {
      const int r = min(rbase + j, B - 1);
      st[j] = win.start[r];
      ct[j] = win.count[r];
    }
#pragma unroll
    for (int j = 0; j < RPW; ++j)
      if (hq / G == j) {
        wst = st[j];
        wen = st[j] + ct[j];
      }
  }
  // the keys inside every query window of the wave: batches wholly in [wlo, whi) need no per-key mask
  int wlo = wst, whi = wen;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    wlo = max(wlo, __shfl_xor(wlo, o, 64));
    whi = min(whi, __shfl_xor(whi, o, 64));
  }
  const int chunk = (u1 - u0 + nsplit - 1) / nsplit;
  const int k0 = u0 + sp * chunk, k1 = min(u1, k0 + chunk);
  const uint16_t* Kb = K + (size_t)g * cap * HD;  // the shared cache (row 0)

  // first key tile in flight before the q prologue (both parts: registers st0, st1)
  u32x4 st0[2], st1[2];
  const bool any = k0 < k1;
  if (any) {
    mq_load_part(Kb, cap, k1, k0, 0, tid, st0);
    mq_load_part(Kb, cap, k1, k0, 1, tid, st1);
  }

  // q_norm + rotation of the lane's query: the lane holds dims 32 s + 8 kq + e (s < 8, e < 8); the rotation partner
  // of dim d < 128 is d + 128, the same lane's step s + 4; the norm's sum spans the four lanes of the query (kq)
  uint4 qhi[KSTEPS], qlo[KSTEPS];
  {
    const float* qr = q + ((size_t)rq * nh + head) * HD + 8 * kq;
    const float* tab = rope + ((size_t)rq * 2 + type) * 2 * half + 8 * kq;
    float4 qv[KSTEPS][2], co[4][2], si[4][2];
    uint4 qw[KSTEPS];
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      qv[s][0] = *reinterpret_cast<const float4*>(qr + 32 * s);
      qv[s][1] = *reinterpret_cast<const float4*>(qr + 32 * s + 4);
      qw[s] = *reinterpret_cast<const uint4*>(qnorm + 32 * s + 8 * kq);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      co[s][0] = *reinterpret_cast<const float4*>(tab + 32 * s);
      co[s][1] = *reinterpret_cast<const float4*>(tab + 32 * s + 4);
      si[s][0] = *reinterpret_cast<const float4*>(tab + half + 32 * s);
      si[s][1] = *reinterpret_cast<const float4*>(tab + half + 32 * s + 4);
    }
    float v[KSTEPS][8];
    float ss = 0.f;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      const float f[8] = {qv[s][0].x, qv[s][0].y, qv[s][0].z, qv[s][0].w,
                          qv[s][1].x, qv[s][1].y, qv[s][1].z, qv[s][1].w};
      float w8[8];
      unpack8(qw[s], w8);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        v[s][e] = f[e] * w8[e];
        ss = fmaf(f[e], f[e], ss);
      }
    }
    ss += xr_partner<16>(ss);
    ss += xr_partner<32>(ss);
    const float rn = rsqrt_hw(ss / (float)HD + eps);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const float c8[8] = {co[s][0].x, co[s][0].y, co[s][0].z, co[s][0].w, co[s][1].x, co[s][1].y, co[s][1].z, co[s][1].w};
      const float s8[8] = {si[s][0].x, si[s][0].y, si[s][0].z, si[s][0].w, si[s][1].x, si[s][1].y, si[s][1].z, si[s][1].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float lo = v[s][e] * rn, hi = v[s + 4][e] * rn;
        v[s][e] = lo * c8[e] - hi * s8[e];
        v[s + 4][e] = hi * c8[e] + lo * s8[e];
      }
    }
    // the softmax scale (with log2 e) goes into q before the split, so the products are the exponents' arguments
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      uint32_t h32[4], l32[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        split_bf16x2(v[s][2 * e] * scale_log2, v[s][2 * e + 1] * scale_log2, h32[e], l32[e]);
      qhi[s] = make_uint4(h32[0], h32[1], h32[2], h32[3]);
      qlo[s] = make_uint4(l32[0], l32[1], l32[2], l32[3]);
    }
  }

  float mrun = -INFINITY, lrun = 0.f;  // softmax state of query hq (identical in its four lanes)
  f32x4 acc[TILES];
#pragma unroll
  for (int t = 0; t < TILES; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (any) {
    mq_store_part(&kt[0][0][0], 0, tid, st0);
    mq_store_part(&kt[0][0][0], 1, tid, st1);
#pragma unroll
    for (int p = 2; p < KT / 32; p += 2) {  // the rest of a longer first tile
      mq_load_part(Kb, cap, k1, k0, p, tid, st0);
      mq_load_part(Kb, cap, k1, k0, p + 1, tid, st1);
      mq_store_part(&kt[0][0][0], p, tid, st0);
      mq_store_part(&kt[0][0][0], p + 1, tid, st1);
    }
  }
  __syncthreads();
  int buf = 0;
  for (int tb = k0; tb < k1; tb += KT) {  // block-uniform
    const bool more = tb + KT < k1;
    // the next tile, in 32-key parts, into the other buffer (free since the last barrier): each part's loads are in
    // flight during one 32-key batch, and at most two parts' registers are live at a time
    if (more) mq_load_part(Kb, cap, k1, tb + KT, 0, tid, st0);
#pragma unroll
    for (int j = 0; j < KT / 32; ++j) {  // 32-key batches: two score tiles, one softmax update
      const int kb = tb + 32 * j;
      if (kb < k1) {  // block-uniform
      f32x4 sacc[2];
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        // K operands read two steps ahead of the products
        const uint16_t* krow = &kt[buf][32 * j + 16 * h2 + hq][8 * (kq ^ mq_swz(hq))];
        uint4 kcur = *reinterpret_cast<const uint4*>(krow);
        uint4 knx = *reinterpret_cast<const uint4*>(krow + 32);
        sacc[h2] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KSTEPS; ++s) {
          const uint4 knext = knx;
          knx = *reinterpret_cast<const uint4*>(krow + 32 * min(s + 2, KSTEPS - 1));
          const bf16x8 a = __builtin_bit_cast(bf16x8, kcur);
          sacc[h2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, qhi[s]), sacc[h2], 0, 0, 0);
          sacc[h2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, qlo[s]), sacc[h2], 0, 0, 0);
          kcur = knext;
        }
      }
      // scores S[query hq][key kb + 16 h2 + 4 kq + r], masked to the query row's window
      float sv[8];
      const bool inside = kb >= wlo && kb + 32 <= whi && kb + 32 <= k1;  // wave-uniform: no key of the batch masked
      if (inside) {
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
          for (int r = 0; r < 4; ++r) sv[4 * h2 + r] = sacc[h2][r];
      } else {
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int t = kb + 16 * h2 + 4 * kq + r;
            sv[4 * h2 + r] = (t < k1 && t >= wst && t < wen) ? sacc[h2][r] : -INFINITY;
          }
      }
      float mt = sv[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) mt = fmaxf(mt, sv[i]);
      mt = fmaxf(mt, xr_partner<16>(mt));
      mt = fmaxf(mt, xr_partner<32>(mt));
      // the reference maximum moves only when a score exceeds it by more than 2^8: below that the weights stay under
      // 256, far inside fp32 and kept to fp32-level accuracy by the bf16 hi + lo split, and most batches skip the
      // rescale of the 64 output sums
      const float mn = (mt > mrun + 8.0f) ? mt : mrun;
      // 2^x on the hardware instruction: weights below 2^-126 flush to zero, far below what a weight contributes, and
      // 2^-inf is 0, so masked keys and a first maximum need no select: only a query with no key yet (mn = -inf)
      // takes 0 as its reference, which leaves its weights and alpha at 0
      const float mref = (mn == -INFINITY) ? 0.f : mn;
      const float alpha = __builtin_amdgcn_exp2f(mrun - mref);
      float pv[8], ps = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        pv[i] = __builtin_amdgcn_exp2f(sv[i] - mref);
        ps += pv[i];
      }
      ps += xr_partner<16>(ps);
      ps += xr_partner<32>(ps);
      lrun = lrun * alpha + ps;
      mrun = mn;
      // P as the A operand of v_mfma_f32_16x16x32_bf16 over the 32 keys: lane l supplies k = 8 kq + i, which stands
      // for key 4 kq + i (i < 4) and key 16 + 4 kq + (i - 4); the V operand below follows the same order
      uint32_t ph[4], pl[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) split_bf16x2(pv[2 * i], pv[2 * i + 1], ph[i], pl[i]);
      const uint4 phi = make_uint4(ph[0], ph[1], ph[2], ph[3]);
      const uint4 plo = make_uint4(pl[0], pl[1], pl[2], pl[3]);
      // rescale only when some query's maximum moved (alpha is exactly 1 otherwise); output rows are queries
      // 4 kq + r, whose alphas live in lanes 4 kq + r
      if (__any(alpha != 1.0f)) {
        float al[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float a0 = readlane_f(alpha, r), a1 = readlane_f(alpha, 4 + r);
          const float a2 = readlane_f(alpha, 8 + r), a3 = readlane_f(alpha, 12 + r);
          al[r] = kq == 0 ? a0 : (kq == 1 ? a1 : (kq == 2 ? a2 : a3));
        }
#pragma unroll
        for (int t = 0; t < TILES; ++t)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[t][r] *= al[r];
      }
      // V operand: keys 32 j + 4 kq + r and 32 j + 16 + 4 kq + r of dim 16 t + hq, two transposing reads of the
      // 4 x 16 blocks at those key rows
      const uint16_t* vrow =
          &kt[buf][32 * j + 4 * kq + (hq >> 2)][8 * (((hq & 3) >> 1) ^ mq_swz(4 * kq)) + 4 * (hq & 1)];
#pragma unroll
      for (int t = 0; t < TILES; ++t) {
        const i16x4 v0 = lds_read_tr16(vrow + 16 * t);
        const i16x4 v1 = lds_read_tr16(vrow + 16 * LROW + 16 * t);
        const bf16x8 vb = __builtin_bit_cast(bf16x8, (i16x8){v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]});
        f32x4 a = acc[t];
        a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, phi), vb, a, 0, 0, 0);
        a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, plo), vb, a, 0, 0, 0);
        acc[t] = a;
      }
      }
      if (more) {  // part j of the next tile to LDS, part j + 1 into the freed registers
        if ((j & 1) == 0) {
          mq_store_part(&kt[buf ^ 1][0][0], j, tid, st0);
          if (j + 1 < KT / 32) mq_load_part(Kb, cap, k1, tb + KT, j + 1, tid, st1);
        } else {
          mq_store_part(&kt[buf ^ 1][0][0], j, tid, st1);
          if (j + 1 < KT / 32) mq_load_part(Kb, cap, k1, tb + KT, j + 1, tid, st0);
        }
      }
    }
    __syncthreads();
    buf ^= 1;
  }
  // outputs: query 4 kq + r of the wave holds dims 16 t + hq in acc[t][r]; its (max, sum) is in lane 4 kq + r
  float Lq[4];
  bool live[4];
  size_t obase[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int qq = 4 * kq + r;
    const float l0 = readlane_f(lrun, r), l1 = readlane_f(lrun, 4 + r), l2 = readlane_f(lrun, 8 + r),
                l3 = readlane_f(lrun, 12 + r);
    Lq[r] = kq == 0 ? l0 : (kq == 1 ? l1 : (kq == 2 ? l2 : l3));
    const int row = rbase + qq / G;
    live[r] = row < B;
    obase[r] = (size_t)min(row, B - 1) * nh + g * G + qq % G;  // (row, head) index
  }
#pragma unroll
  for (int t = 0; t < TILES; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (!live[r]) continue;
      const int d = 16 * t + hq;
      if (nsplit == 1) {
        o[obase[r] * HD + d] = (Lq[r] > 0.f) ? acc[t][r] / Lq[r] : 0.f;
      } else {
        pacc[(obase[r] * kMaxSplit + sp) * HD + d] = acc[t][r];
      }
    }
  if (nsplit > 1 && kq == 0 && qlive) {
    const size_t slot = ((size_t)rq * nh + head) * kMaxSplit + sp;
    pml[slot * 2 + 0] = mrun;
    pml[slot * 2 + 1] = lrun;
  }
}

}  // namespace

hipError_t launch_attn_shared(hipStream_t s, int B, int nh, int nkv, const float* q, const uint16_t* qnorm, float eps,
                              const float* rope, int type, const uint16_t* K, int cap, const RowWindows& win,
                              int nsplit, float scale_log2, float* pacc, float* pml, float* o) {
  const int G = nh / nkv;
  // the union of the rows' windows
  int u0 = win.start[0], u1 = win.start[0] + win.count[0];
  for (int b = 1; b < B; ++b) {
    u0 = win.start[b] < u0 ? win.start[b] : u0;
    u1 = win.start[b] + win.count[b] > u1 ? win.start[b] + win.count[b] : u1;
  }
  const dim3 grid(nsplit, (B + 8 * (16 / G) - 1) / (8 * (16 / G)), nkv);
#define MTPD_MQ(G_)                                                                                              \
  if (G == G_)                                                                                                   \
    return go(k_attn_mq<G_>, grid, 512, 0, s, B, nh, nkv, q, qnorm, eps, rope, type, K, cap, win, nsplit, u0, u1, \
              scale_log2, pacc, pml, o);
  MTPD_MQ(1) MTPD_MQ(2) MTPD_MQ(4) MTPD_MQ(8)
#undef MTPD_MQ
  return hipErrorInvalidValue;
}

}  // namespace mtpd
