// Single-query attention over the shared caches: the vector-ALU kernel (any head_dim in {64, 128, 256}) and the
// matrix-core kernel (head_dim 256, up to 8 query heads per kv head); caches shared by all rows go to the
// multi-query kernel of k_attention_shared.hip.
//
// Pages cited (by title; sections as headed on each page):
//   [MTP doc]    "Gemma 4 Multi-Token Prediction (MTP) drafter" (llama.cpp fork, gemma4-assistant.md)
//   [Inventory]  "Gemma 4 Assistant (MTP drafter) - tensor inventory (Stage 0)"
//   [Guide]      "Gemma 4 Assistant 使用指南：用 MTP 投机解码与 KV Sharing 加速 Gemma 4 推理" (gitcode blog)
#include "attn_mfma.h"

namespace mtpd {
namespace {

// ------------------------------------------------------------------------------------------------------------
// single-query attention over the shared cache ([MTP doc] "What it is": Q-only attention on the target's
// last-layer K/V; [Guide] section 2(4); [Inventory] "Notes for llama.cpp port" 2: V taken from K)
// grid (nsplit, B * nkv), NW waves per block. HD = head_dim, G = query heads per kv head, DPL = dims per lane,
// KB = keys per batch (KB * G = 64 scores, one per lane after the transpose-reduction).

template <int DPL>
struct RawT;
template <>
struct RawT<4> { using T = uint2; };
template <>
struct RawT<2> { using T = uint32_t; };
template <>
struct RawT<1> { using T = uint16_t; };

template <int DPL>
__device__ __forceinline__ void unpack_raw(const typename RawT<DPL>::T& r, float* f) {
  if constexpr (DPL == 4) {
    f[0] = bf_lo(r.x); f[1] = bf_hi(r.x); f[2] = bf_lo(r.y); f[3] = bf_hi(r.y);
  } else if constexpr (DPL == 2) {
    f[0] = bf_lo(r); f[1] = bf_hi(r);
  } else {
    f[0] = bf2f(r);
  }
}

template <int HD, int G, int NW>
__global__ __launch_bounds__(NW * 64) void k_attn(int B, int nh, int nkv, const float* __restrict__ q,
                                                  const uint16_t* __restrict__ qnorm, float eps,
                                                  const float* __restrict__ rope, int type,
                                                  const uint16_t* __restrict__ K, const uint16_t* __restrict__ Vc,
                                                  int cap, RowWindows win, int nsplit, float scale_log2,
                                                  float* __restrict__ pacc, float* __restrict__ pml,
                                                  float* __restrict__ o) {
  constexpr int DPL = HD / 64;
  constexpr int KB = 64 / G;
  using Raw = typename RawT<DPL>::T;
  __shared__ float qs[G][HD];
  __shared__ float wml[NW][G][2];
  __shared__ float wacc[NW][G][HD];
  const int sp = blockIdx.x, bg = blockIdx.y;
  const int b = bg / nkv, g = bg % nkv;
  const int wave = wave_id(), lane = lane_id();
  constexpr int half = HD / 2;

  const int cntk = win.count[b];
  const int chunk = (cntk + nsplit - 1) / nsplit;
  const int k0 = win.start[b] + sp * chunk;
  const int k1 = min(win.start[b] + cntk, k0 + chunk);
  const bool same_v = (Vc == K);
  const size_t crow = win.shared ? 0 : (size_t)b;  // cache row (shared caches: row 0 for every batch row)
  const uint16_t* Kb = K + (crow * nkv + g) * (size_t)cap * HD + lane * DPL;
  const uint16_t* Vb = Vc + (crow * nkv + g) * (size_t)cap * HD + lane * DPL;
  // first batch of keys in flight before the q prologue
  Raw kcur[KB], knext[KB];
  int t0 = k0 + wave * KB;
  if (t0 < k1) {
#pragma unroll
    for (int j = 0; j < KB; ++j) kcur[j] = *reinterpret_cast<const Raw*>(Kb + (size_t)slot_of(min(t0 + j, k1 - 1), cap) * HD);
  }

  // q_norm + rotation at the row's constant position ([Guide] section 2(2))
  const float* tab = rope + ((size_t)b * 2 + type) * 2 * half;
  for (int hh = wave; hh < G; hh += NW) {
    const float* qr = q + ((size_t)b * nh + g * G + hh) * HD;
    float v[DPL], wq[DPL], co[DPL], si[DPL];
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) {
      const int d = lane * DPL + e;
      const int i = d & (half - 1);
      v[e] = qr[d];
      wq[e] = bf2f(qnorm[d]);
      co[e] = tab[i];
      si[e] = tab[half + i];
      ss = fmaf(v[e], v[e], ss);
    }
    ss = wave_sum(ss);
    const float r = rsqrt_hw(ss / (float)HD + eps);
#pragma unroll
    for (int e = 0; e < DPL; ++e) v[e] = v[e] * r * wq[e];
#pragma unroll
    for (int e = 0; e < DPL; ++e) {
      const float partner = __shfl_xor(v[e], 32, 64);  // dim i <-> i + HD/2
      qs[hh][lane * DPL + e] = (lane < 32) ? (v[e] * co[e] - partner * si[e]) : (v[e] * co[e] + partner * si[e]);
    }
  }
  __syncthreads();
  float qr[G][DPL];
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
#pragma unroll
    for (int e = 0; e < DPL; ++e) qr[hh][e] = qs[hh][lane * DPL + e];

  float mrun[G], lrun[G], acc[G][DPL];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    mrun[hh] = -INFINITY;
    lrun[hh] = 0.f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[hh][e] = 0.f;
  }
  const int jl = lane / G, hl = lane % G;

  for (; t0 < k1; t0 += NW * KB) {
    const int nk = min(KB, k1 - t0);
    const int tn = t0 + NW * KB;
    if (tn < k1) {  // next batch in flight while this one is computed
#pragma unroll
      for (int j = 0; j < KB; ++j) knext[j] = *reinterpret_cast<const Raw*>(Kb + (size_t)slot_of(min(tn + j, k1 - 1), cap) * HD);
    }
    float sc[64];
#pragma unroll
    for (int j = 0; j < KB; ++j) {
      float kf[DPL];
      unpack_raw<DPL>(kcur[j], kf);
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < DPL; ++e) s = fmaf(kf[e], qr[hh][e], s);
        sc[j * G + hh] = s;
      }
    }
    XR<64, 32>::run(sc, lane);  // lane l: score of key l / G, head l % G
    const float s = (jl < nk) ? sc[0] * scale_log2 : -INFINITY;
    float mx = s;
#pragma unroll
    for (int of = G; of < 64; of <<= 1) mx = fmaxf(mx, __shfl_xor(mx, of, 64));
    float alpha[G];
    float mhl = 0.f;
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      const float mn = fmaxf(mrun[hh], readlane_f(mx, hh));
      alpha[hh] = (mrun[hh] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mrun[hh] - mn);
      mrun[hh] = mn;
      mhl = (hl == hh) ? mn : mhl;
    }
    const float p = (jl < nk) ? __builtin_amdgcn_exp2f(s - mhl) : 0.f;
    float ps = p;
#pragma unroll
    for (int of = G; of < 64; of <<= 1) ps += __shfl_xor(ps, of, 64);
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      lrun[hh] = lrun[hh] * alpha[hh] + readlane_f(ps, hh);
#pragma unroll
      for (int e = 0; e < DPL; ++e) acc[hh][e] *= alpha[hh];
    }
    // P.V (p of masked keys is 0)
    Raw vraw[KB];
    if (!same_v) {
#pragma unroll
      for (int j = 0; j < KB; ++j) vraw[j] = *reinterpret_cast<const Raw*>(Vb + (size_t)slot_of(min(t0 + j, k1 - 1), cap) * HD);
    }
#pragma unroll
    for (int j = 0; j < KB; ++j) {
      float vf[DPL];
      unpack_raw<DPL>(same_v ? kcur[j] : vraw[j], vf);
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        const float pj = readlane_f(p, j * G + hh);
#pragma unroll
        for (int e = 0; e < DPL; ++e) acc[hh][e] = fmaf(pj, vf[e], acc[hh][e]);
      }
    }
#pragma unroll
    for (int j = 0; j < KB; ++j) kcur[j] = knext[j];
  }
  // combine the waves of this block
  if (lane == 0) {
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      wml[wave][hh][0] = mrun[hh];
      wml[wave][hh][1] = lrun[hh];
    }
  }
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
#pragma unroll
    for (int e = 0; e < DPL; ++e) wacc[wave][hh][lane * DPL + e] = acc[hh][e];
  __syncthreads();
  for (int i = threadIdx.x; i < G * HD; i += NW * 64) {
    const int hh = i / HD, d = i % HD;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, wml[w][hh][0]);
    float L = 0.f, A = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float mw = wml[w][hh][0];
        const float f = (mw == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mw - M);
        L = fmaf(wml[w][hh][1], f, L);
        A = fmaf(wacc[w][hh][d], f, A);
      }
    }
    const size_t hq = (size_t)b * nh + g * G + hh;
    if (nsplit == 1) {
      o[hq * HD + d] = (L > 0.f) ? A / L : 0.f;
    } else {
      const size_t slot = hq * kMaxSplit + sp;
      pacc[slot * HD + d] = A;
      if (d == 0) {
        pml[slot * 2 + 0] = M;
        pml[slot * 2 + 1] = L;
      }
    }
  }
}

// Matrix-core variant for head_dim 256 and up to 8 query heads per kv head. Per wave and batch of 16 keys:
//   S[16 keys][16 columns] = K_tile . [q_hi | q_lo]^T with v_mfma_f32_16x16x32_bf16: the key rows load straight into
//     the A operand (lane l: key l%16, 8 dims at 8*(l/16) of each 32-dim step); the fp32 query is split into two
//     bf16 terms q = q_hi + q_lo (relative error <= 2^-16) so the product keeps fp32-level accuracy: column h holds
//     q_hi of head h, column 8 + h its q_lo, and one exchange 8 lanes apart sums the two;
//   online softmax on the S layout (lane l holds keys 4*(l/16)+r of head l%16);
//   O[16 rows][256] += P . V with v_mfma_f32_16x16x16_bf16: P split into bf16 hi (row h) + lo (row 8 + h) is already
//     in the A layout, V comes from the wave's LDS copy of the key tile, read column-wise by transposing LDS reads (4
//     keys of one dim per lane); the lo rows are folded into the hi rows once, after the last batch.

template <int G, int NW>
__global__ __launch_bounds__(NW * 64, 2) void k_attn_mfma(int B, int nh, int nkv, const float* __restrict__ q,
                                                          const uint16_t* __restrict__ qnorm, float eps,
                                                          const float* __restrict__ rope, int type,
                                                          const uint16_t* __restrict__ K,
                                                          const uint16_t* __restrict__ Vc, int cap, RowWindows win,
                                                          int nsplit, float scale_log2, float* __restrict__ pacc,
                                                          float* __restrict__ pml, float* __restrict__ o) {
  constexpr int HD = 256, KSTEPS = HD / 32, TILES = HD / 16, LROW = HD + 8, S = NW * 16;
  static_assert(G == 1 || G == 2 || G == 4 || G == 8, "the heads of a kv group sit in lanes 0..G-1 of the score tile");
  constexpr int GQ = (G + 3) / 4;      // 4-head row groups of the output tile that hold real heads
  constexpr int HPW = (G + NW - 1) / NW;  // heads whose q a wave normalises and rotates
  // the q staging buffer is dead once the B operands are built (a barrier later), so the combine reuses it
  constexpr int QS_FLOATS = G * HD, WACC_FLOATS = NW * HD * 4 * GQ;
  __shared__ __attribute__((aligned(16))) float qs_wacc[QS_FLOATS > WACC_FLOATS ? QS_FLOATS : WACC_FLOATS];
  float (*qs)[HD] = reinterpret_cast<float (*)[HD]>(qs_wacc);                  // [head][dim]
  float (*wacc)[HD][4 * GQ] = reinterpret_cast<float (*)[HD][4 * GQ]>(qs_wacc);  // [wave][dim][head]
  // [step][hi/lo][head slot][kq][8 dims]; slots G .. 7 stay zero (the unused columns of the score tile)
  __shared__ __attribute__((aligned(16))) uint16_t qop[KSTEPS][2][8][4][8];
  __shared__ __attribute__((aligned(16))) uint16_t vt[NW][16][LROW];
  __shared__ __attribute__((aligned(16))) float wml[NW][G][2];
  static_assert(NW * 64 == HD, "one thread per dim in the combine");
  const int sp = blockIdx.x, bg = blockIdx.y;
  const int b = bg / nkv, g = bg % nkv;
  const int wave = wave_id(), lane = lane_id();
  const int hq = lane & 15, kq = lane >> 4;
  constexpr int half = HD / 2;

  const int cntk = win.count[b];
  const int chunk = (cntk + nsplit - 1) / nsplit;
  const int k0 = win.start[b] + sp * chunk;
  const int k1 = min(win.start[b] + cntk, k0 + chunk);
  const bool same_v = (Vc == K);
  const size_t crow = win.shared ? 0 : (size_t)b;  // cache row (shared caches: row 0 for every batch row)
  const uint16_t* Kb = K + (crow * nkv + g) * (size_t)cap * HD + 8 * kq;
  const uint16_t* Vb = Vc + (crow * nkv + g) * (size_t)cap * HD + 8 * kq;

  // inputs of q_norm + rotation first (waits count loads in issue order, so these must precede the key batch)
  const float* tab = rope + ((size_t)b * 2 + type) * 2 * half;
  // the wave's heads wave + NW j (waves beyond G repeat the last head and store nothing)
  float4 qv[HPW];
#pragma unroll
  for (int j = 0; j < HPW; ++j)
    qv[j] = *reinterpret_cast<const float4*>(q + ((size_t)b * nh + g * G + min(wave + NW * j, G - 1)) * HD + lane * 4);
  const uint2 qw = *reinterpret_cast<const uint2*>(qnorm + lane * 4);
  const int i0 = (lane * 4) & (half - 1);
  const float4 co4 = *reinterpret_cast<const float4*>(tab + i0);
  const float4 si4 = *reinterpret_cast<const float4*>(tab + half + i0);
  __builtin_amdgcn_sched_barrier(0);

  // key rows of batch t (lane: key t + hq, dims 32c + 8kq .. +8), clamped into the block's range; batch t + S is
  // in flight while batch t is computed
  uint4 ka[KSTEPS], kn[KSTEPS];
  int t0 = k0 + wave * 16;
  {
    const uint16_t* r = Kb + (size_t)slot_of(min(t0 + hq, k1 - 1), cap) * HD;
#pragma unroll
    for (int c = 0; c < KSTEPS; ++c) ka[c] = *reinterpret_cast<const uint4*>(r + 32 * c);
  }
  __builtin_amdgcn_sched_barrier(0);  // the q arithmetic below must not be hoisted above the key loads

  // q_norm + rotation at the row's constant position ([Guide] section 2(2)); lane l holds dims 4l .. 4l+3, whose
  // rotation partners (dim i <-> i + HD/2) sit in lane l ^ 32
#pragma unroll
  for (int j = 0; j < HPW; ++j) {
    const int hh = wave + NW * j;
    float v[4] = {qv[j].x, qv[j].y, qv[j].z, qv[j].w}, wq[4];
    const float co[4] = {co4.x, co4.y, co4.z, co4.w}, si[4] = {si4.x, si4.y, si4.z, si4.w};
    unpack4(qw, wq);
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) ss = fmaf(v[e], v[e], ss);
    ss = wave_sum(ss);
    const float r = rsqrt_hw(ss / (float)HD + eps);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = v[e] * r * wq[e];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float partner = xr_partner<32>(v[e]);
      const float rot = (lane < 32) ? (v[e] * co[e] - partner * si[e]) : (v[e] * co[e] + partner * si[e]);
      if (hh < G) qs[hh][lane * 4 + e] = rot;
    }
  }
  __syncthreads();
  // q = q_hi + q_lo in bf16, stored in the MFMA B-operand order
  for (int i = threadIdx.x; i < KSTEPS * 8 * 4 * 8; i += NW * 64) {
    const int e = i & 7, kk = (i >> 3) & 3, hh = (i >> 5) & 7, c = i >> 8;
    const float v = hh < G ? qs[hh][32 * c + 8 * kk + e] : 0.f;
    const uint16_t hb = f2bf(v);
    qop[c][0][hh][kk][e] = hb;
    qop[c][1][hh][kk][e] = f2bf(v - bf2f(hb));
  }
  __syncthreads();

  float mrun = -INFINITY, lrun = 0.f;  // softmax state of head hq (identical in the 4 lanes of that head)
  f32x4 acc[TILES];
#pragma unroll
  for (int t = 0; t < TILES; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  uint16_t* tile = &vt[wave][0][0];
  static_assert(S == 64, "mfma_batch takes 16 keys per wave and 4 waves");

  for (; t0 + S < k1; t0 += S)
    mfma_batch<G, true>(t0, k1, Kb, Vb, cap, same_v, scale_log2, tile, qop, ka, kn, acc, mrun, lrun);
  if (t0 < k1) mfma_batch<G, false>(t0, k1, Kb, Vb, cap, same_v, scale_log2, tile, qop, ka, kn, acc, mrun, lrun);
  attn_fold_rows(acc);
  // combine the waves of this block: head h's softmax state is in lane h; output row group kq (heads 4kq .. +3)
  // sits in lanes 16kq .. +15: dim 16t + hq, heads in the four registers of acc[t], stored as one float4 per dim
  if (lane < G) {
    wml[wave][lane][0] = mrun;
    wml[wave][lane][1] = lrun;
  }
  // (the combine buffer overlays the q staging buffer, whose last reads precede the barrier before the key loop)
  if (kq < GQ) {
#pragma unroll
    for (int t = 0; t < TILES; ++t) *reinterpret_cast<f32x4*>(&wacc[wave][16 * t + hq][4 * kq]) = acc[t];
  }
  __syncthreads();
  {
    // thread d: dim d of the G heads over the NW waves
    const int d = threadIdx.x;
    f32x4 av[NW][GQ];
    float2 ml[NW][G];
#pragma unroll
    for (int w = 0; w < NW; ++w) {
#pragma unroll
      for (int j = 0; j < GQ; ++j) av[w][j] = *reinterpret_cast<const f32x4*>(&wacc[w][d][4 * j]);
#pragma unroll
      for (int hh = 0; hh < G; ++hh) ml[w][hh] = *reinterpret_cast<const float2*>(&wml[w][hh][0]);
    }
    asm volatile("" ::: "memory");  // all LDS reads issued before the arithmetic
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < NW; ++w) M = fmaxf(M, ml[w][hh].x);
      float L = 0.f, A = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float mw = ml[w][hh].x;
        const float f = (mw == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mw - M);
        L = fmaf(ml[w][hh].y, f, L);
        A = fmaf(av[w][hh >> 2][hh & 3], f, A);
      }
      const size_t hqq = (size_t)b * nh + g * G + hh;
      if (nsplit == 1) {
        o[hqq * HD + d] = (L > 0.f) ? A / L : 0.f;
      } else {
        const size_t slot = hqq * kMaxSplit + sp;
        pacc[slot * HD + d] = A;
        if (d == 0) {
          pml[slot * 2 + 0] = M;
          pml[slot * 2 + 1] = L;
        }
      }
    }
  }
}

}  // namespace

// ------------------------------------------------------------------------------------------------------------
// launcher

bool attn_uses_multi_query(bool valu, bool shared, int hd, bool same_v) { return shared && hd == 256 && same_v && !valu; }

hipError_t launch_attn(hipStream_t s, bool valu, int B, int nh, int nkv, int hd, const float* q, const uint16_t* qnorm,
                       float eps, const float* rope, int type, const uint16_t* K, const uint16_t* V, int cap,
                       const RowWindows& win, int nsplit, float scale, float* pacc, float* pml, float* o) {
  dim3 grid(nsplit, B * nkv);
  const float sl2 = scale * 1.4426950408889634f;
  const int G = nh / nkv;
  if (attn_uses_multi_query(valu, win.shared != 0, hd, V == K))
    return launch_attn_shared(s, B, nh, nkv, q, qnorm, eps, rope, type, K, cap, win, nsplit, sl2, pacc, pml, o);
  if (hd == 256 && G <= 8 && !valu) {
    if (G == 8) return go(k_attn_mfma<8, 4>, grid, 256, 0, s, B, nh, nkv, q, qnorm, eps, rope, type, K, V, cap, win, nsplit, sl2, pacc, pml, o);
    if (G == 4) return go(k_attn_mfma<4, 4>, grid, 256, 0, s, B, nh, nkv, q, qnorm, eps, rope, type, K, V, cap, win, nsplit, sl2, pacc, pml, o);
    if (G == 2) return go(k_attn_mfma<2, 4>, grid, 256, 0, s, B, nh, nkv, q, qnorm, eps, rope, type, K, V, cap, win, nsplit, sl2, pacc, pml, o);
    return go(k_attn_mfma<1, 4>, grid, 256, 0, s, B, nh, nkv, q, qnorm, eps, rope, type, K, V, cap, win, nsplit, sl2, pacc, pml, o);
  }
#define MTPD_ATTN(HD_, G_, NW_)                                                                             \
  if (hd == HD_ && G == G_) {                                                                               \
    return go(k_attn<HD_, G_, NW_>, grid, NW_ * 64, 0, s, B, nh, nkv, q, qnorm, eps, rope, type, K, V, cap, \
              win, nsplit, sl2, pacc, pml, o);                                                              \
  }
  if (nsplit == 1) {
    MTPD_ATTN(256, 1, 8) MTPD_ATTN(256, 2, 8) MTPD_ATTN(256, 4, 8) MTPD_ATTN(256, 8, 4)
    MTPD_ATTN(128, 1, 8) MTPD_ATTN(128, 2, 8) MTPD_ATTN(128, 4, 8) MTPD_ATTN(128, 8, 8)
    MTPD_ATTN(64, 1, 8) MTPD_ATTN(64, 2, 8) MTPD_ATTN(64, 4, 8) MTPD_ATTN(64, 8, 8)
  } else {
    MTPD_ATTN(256, 1, 4) MTPD_ATTN(256, 2, 4) MTPD_ATTN(256, 4, 4) MTPD_ATTN(256, 8, 4)
    MTPD_ATTN(128, 1, 4) MTPD_ATTN(128, 2, 4) MTPD_ATTN(128, 4, 4) MTPD_ATTN(128, 8, 4)
    MTPD_ATTN(64, 1, 4) MTPD_ATTN(64, 2, 4) MTPD_ATTN(64, 4, 4) MTPD_ATTN(64, 8, 4)
  }
#undef MTPD_ATTN
  return hipErrorInvalidValue;
}

}  // namespace mtpd
