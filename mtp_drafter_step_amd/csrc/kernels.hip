// Drafter-step kernels for gfx950 (CDNA4, wave64).
//
// Pages cited (by title; sections as headed on each page):
//   [MTP doc]    "Gemma 4 Multi-Token Prediction (MTP) drafter" (llama.cpp fork, gemma4-assistant.md)
//   [Inventory]  "Gemma 4 Assistant (MTP drafter) - tensor inventory (Stage 0)"
//   [Guide]      "Gemma 4 Assistant 使用指南：用 MTP 投机解码与 KV Sharing 加速 Gemma 4 推理" (gitcode blog)
//
// Numerics: bf16 storage, fp32 activations and accumulation; integer decisions (top-k, argmax) on fp32 values
// with ties to the lower index.
//
// Dense kernels: a block owns a tile of outputs for a group of 4 batch rows; each wave computes a few outputs for
// the 4 rows with lanes striding the reduction dimension, then a butterfly transpose-reduction leaves one finished
// (row, output) sum per lane group. Inputs that need a norm are normalised once per block into LDS.
#include "kernels.h"

#include <math.h>

namespace mtpd {

namespace {

constexpr int kRG = kRowGroup;

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// fp32 -> bf16, round to nearest even (finite inputs)
__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// order-preserving map of fp32 onto uint32 (larger float -> larger integer)
__device__ __forceinline__ uint32_t f32_order(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t u64_max(uint64_t a, uint64_t b) { return a > b ? a : b; }

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int o) {
  const uint32_t lo = __shfl_xor((uint32_t)v, o, 64);
  const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), o, 64);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = u64_max(v, shfl_xor_u64(v, o));
  return v;
}

// max over a 256-thread block; every thread gets the result. `red` holds 4 entries.
__device__ __forceinline__ uint64_t block_max_u64(uint64_t v, uint64_t* red) {
  v = wave_max_u64(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return u64_max(u64_max(red[0], red[1]), u64_max(red[2], red[3]));
}

__device__ __forceinline__ float gelu_tanh(float a) {
  const float c = 0.7978845608028654f;  // sqrt(2/pi)
  return 0.5f * a * (1.0f + tanhf(c * (a + 0.044715f * a * a * a)));
}

__device__ __forceinline__ float readlane_f(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// Butterfly transpose-reduction of V per-lane values over the 64 lanes. Afterwards v[0] of lane l holds the
// wave-wide sum of value index (l >> (6 - log2 V)).
template <int V, int O>
struct XR {
  static __device__ __forceinline__ void run(float* v, int lane) {
    if constexpr (V > 1) {
      constexpr int H = V / 2;
      const bool up = (lane & O) != 0;
#pragma unroll
      for (int i = 0; i < H; ++i) {
        const float send = up ? v[i] : v[i + H];
        const float keep = up ? v[i + H] : v[i];
        v[i] = keep + __shfl_xor(send, O, 64);
      }
      if constexpr (O > 1) XR<H, O / 2>::run(v, lane);
    } else {
      v[0] += __shfl_xor(v[0], O, 64);
      if constexpr (O > 1) XR<1, O / 2>::run(v, lane);
    }
  }
};

template <int V>
__device__ __forceinline__ constexpr int ilog2() {
  return V <= 1 ? 0 : 1 + ilog2<V / 2>();
}

// Load 8 consecutive bf16 as fp32.
__device__ __forceinline__ void load8(const uint16_t* p, float* f) {
  const uint4 w = *reinterpret_cast<const uint4*>(p);
  f[0] = bf_lo(w.x); f[1] = bf_hi(w.x); f[2] = bf_lo(w.y); f[3] = bf_hi(w.y);
  f[4] = bf_lo(w.z); f[5] = bf_hi(w.z); f[6] = bf_lo(w.w); f[7] = bf_hi(w.w);
}

// Residual update + RMSNorm for the block's row group into LDS xs[kRG][H]; one wave per row.
// Rows beyond B are zero. The block with blockIdx.x == 0 stores x_new when res.x_new is set.
__device__ void prologue_norm(const Residual& res, const uint16_t* w_norm, float eps, int B, int H, float* xs) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = blockIdx.y * kRG + wave;
  float* xr = xs + wave * H;
  if (row >= B) {
    for (int i = lane; i < H; i += 64) xr[i] = 0.f;
    return;
  }
  const float* xo = res.x_old + (size_t)row * H;
  float sd = 1.f;
  if (res.delta) {
    const float* dr = res.delta + (size_t)row * H;
    float ss = 0.f;
    for (int i = lane; i < H; i += 64) ss += dr[i] * dr[i];
    ss = wave_sum(ss);
    const float r = 1.0f / sqrtf(ss / (float)H + eps);
    float s2 = 0.f;
    for (int i = lane; i < H; i += 64) {
      const float v = (xo[i] + dr[i] * r * bf2f(res.w_delta[i])) * res.scale;
      xr[i] = v;
      s2 += v * v;
    }
    sd = wave_sum(s2);
  } else {
    float s2 = 0.f;
    for (int i = lane; i < H; i += 64) {
      const float v = xo[i];
      xr[i] = v;
      s2 += v * v;
    }
    sd = wave_sum(s2);
  }
  if (res.x_new && blockIdx.x == 0)
    for (int i = lane; i < H; i += 64) res.x_new[(size_t)row * H + i] = xr[i];
  const float r2 = 1.0f / sqrtf(sd / (float)H + eps);
  for (int i = lane; i < H; i += 64) xr[i] = xr[i] * r2 * bf2f(w_norm[i]);
}

// One wave: y[r][o] = sum_k xs[r][k] * W[n0 + o][k] for r < kRG, o < OPW (fp32 X in LDS, bf16 W in global).
// acc receives the transpose-reduced sums: lane l holds value index (l >> (6 - log2(kRG*OPW))) = r*OPW + o.
template <int OPW>
__device__ __forceinline__ void wave_dense(const float* xs, int ldx, const uint16_t* W, int K, int n0, int N,
                                           float* acc) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < kRG * OPW; ++i) acc[i] = 0.f;
  for (int k = lane * 8; k < K; k += 512) {
    float wf[OPW][8];
#pragma unroll
    for (int o = 0; o < OPW; ++o) {
      if (n0 + o < N) {
        load8(W + (size_t)(n0 + o) * K + k, wf[o]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) wf[o][e] = 0.f;
      }
    }
#pragma unroll
    for (int r = 0; r < kRG; ++r) {
      const float4 a = *reinterpret_cast<const float4*>(xs + r * ldx + k);
      const float4 b = *reinterpret_cast<const float4*>(xs + r * ldx + k + 4);
#pragma unroll
      for (int o = 0; o < OPW; ++o) {
        float s = acc[r * OPW + o];
        s = fmaf(a.x, wf[o][0], s); s = fmaf(a.y, wf[o][1], s); s = fmaf(a.z, wf[o][2], s);
        s = fmaf(a.w, wf[o][3], s); s = fmaf(b.x, wf[o][4], s); s = fmaf(b.y, wf[o][5], s);
        s = fmaf(b.z, wf[o][6], s); s = fmaf(b.w, wf[o][7], s);
        acc[r * OPW + o] = s;
      }
    }
  }
  XR<kRG * OPW, 32>::run(acc, lane);
}

// ------------------------------------------------------------------------------------------------------------
// pre_projection of [target hidden ; embedded token]  ([MTP doc] "What it is": 2x backbone input;
// [Guide] section 2(3))
// grid (H / 4, ceil(B / 4)); each wave one output for the 4 rows.

__global__ __launch_bounds__(256) void k_pre(int B, int Bb, int H, int V, const uint16_t* __restrict__ th,
                                             const int32_t* __restrict__ tok, const uint16_t* __restrict__ emb,
                                             float escale, const uint16_t* __restrict__ W, float* __restrict__ x,
                                             uint32_t* __restrict__ counters, int ncounters) {
  if (blockIdx.x == 0 && blockIdx.y == 0)
    for (int i = threadIdx.x; i < ncounters; i += 256) counters[i] = 0u;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = blockIdx.x * 4 + wave;
  const int r0 = blockIdx.y * kRG;
  const int K = 2 * Bb;
  const uint16_t* hrow[kRG];
  const uint16_t* erow[kRG];
#pragma unroll
  for (int r = 0; r < kRG; ++r) {
    const int b = min(r0 + r, B - 1);
    int t = tok[b];
    t = t < 0 ? 0 : (t >= V ? V - 1 : t);  // out-of-range ids are clamped (documented in the ABI)
    hrow[r] = th + (size_t)b * Bb;
    erow[r] = emb + (size_t)t * Bb;
  }
  float acc[kRG];
#pragma unroll
  for (int r = 0; r < kRG; ++r) acc[r] = 0.f;
  if (n < H) {
    const uint16_t* w = W + (size_t)n * K;
    for (int k = lane * 8; k < K; k += 512) {
      float wf[8];
      load8(w + k, wf);
#pragma unroll
      for (int r = 0; r < kRG; ++r) {
        float xf[8];
        if (k < Bb) {
          load8(hrow[r] + k, xf);
        } else {
          load8(erow[r] + (k - Bb), xf);
          if (escale != 1.0f) {
#pragma unroll
            for (int e = 0; e < 8; ++e) xf[e] *= escale;
          }
        }
        float s = acc[r];
#pragma unroll
        for (int e = 0; e < 8; ++e) s = fmaf(xf[e], wf[e], s);
        acc[r] = s;
      }
    }
  }
  XR<kRG, 32>::run(acc, lane);
  const int idx = lane >> 4;  // row within the group
  if ((lane & 15) == 0 && n < H && r0 + idx < B) x[(size_t)(r0 + idx) * H + n] = acc[0];
}

// ------------------------------------------------------------------------------------------------------------
// q projection ([MTP doc] "Tensor schema": attn_norm, attn_q); grid (QD / 16, ceil(B / 4))

__global__ __launch_bounds__(256) void k_qproj(int B, int H, int QD, Residual res, const uint16_t* __restrict__ w_norm,
                                               float eps, const uint16_t* __restrict__ W, float* __restrict__ q) {
  extern __shared__ float xs[];  // [kRG][H]
  prologue_norm(res, w_norm, eps, B, H, xs);
  __syncthreads();
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n0 = blockIdx.x * 16 + wave * 4;
  float acc[kRG * 4];
  wave_dense<4>(xs, H, W, H, n0, QD, acc);
  const int idx = lane >> 2;  // r * 4 + o
  const int r = blockIdx.y * kRG + (idx >> 2), n = n0 + (idx & 3);
  if ((lane & 3) == 0 && r < B && n < QD) q[(size_t)r * QD + n] = acc[0];
}

// ------------------------------------------------------------------------------------------------------------
// Dense product for o_proj / down: grid (N / 4, ceil(B / 4)); rows of X staged in LDS.

__global__ __launch_bounds__(256) void k_dense(int B, int K, int N, const float* __restrict__ X,
                                               const uint16_t* __restrict__ W, float* __restrict__ y) {
  extern __shared__ float xs[];  // [kRG][K]
  const int r0 = blockIdx.y * kRG;
  for (int i = threadIdx.x; i < kRG * K; i += 256) {
    const int r = i / K, k = i % K;
    xs[i] = (r0 + r < B) ? X[(size_t)(r0 + r) * K + k] : 0.f;
  }
  __syncthreads();
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = blockIdx.x * 4 + wave;
  float acc[kRG];
  wave_dense<1>(xs, K, W, K, n, N, acc);
  const int idx = lane >> 4;
  if ((lane & 15) == 0 && r0 + idx < B && n < N) y[(size_t)(r0 + idx) * N + n] = acc[0];
}

// ------------------------------------------------------------------------------------------------------------
// GeGLU FFN input half ([MTP doc] "Tensor schema": ffn_norm, ffn_gate, ffn_up): grid (F / 16, ceil(B / 4)).
// Each wave: 4 ffn indices x {gate, up} for the 4 rows. Blocks also fill their share of the logits row.

__global__ __launch_bounds__(256) void k_ffn(int B, int H, int F, Residual res, const uint16_t* __restrict__ w_norm,
                                             float eps, const uint16_t* __restrict__ Wg,
                                             const uint16_t* __restrict__ Wu, float* __restrict__ m,
                                             FillRange fill) {
  extern __shared__ float xs[];  // [kRG][H]
  prologue_norm(res, w_norm, eps, B, H, xs);
  __syncthreads();
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int f0 = blockIdx.x * 16 + wave * 4;
  float acc[kRG * 8];
#pragma unroll
  for (int i = 0; i < kRG * 8; ++i) acc[i] = 0.f;
  for (int k = lane * 8; k < H; k += 512) {
    float wg[4][8], wu[4][8];
#pragma unroll
    for (int o = 0; o < 4; ++o) {
      if (f0 + o < F) {
        load8(Wg + (size_t)(f0 + o) * H + k, wg[o]);
        load8(Wu + (size_t)(f0 + o) * H + k, wu[o]);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) wg[o][e] = wu[o][e] = 0.f;
      }
    }
#pragma unroll
    for (int r = 0; r < kRG; ++r) {
      const float4 a = *reinterpret_cast<const float4*>(xs + r * H + k);
      const float4 b = *reinterpret_cast<const float4*>(xs + r * H + k + 4);
      const float xv[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
      for (int o = 0; o < 4; ++o) {
        float sg = acc[r * 8 + o * 2], su = acc[r * 8 + o * 2 + 1];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          sg = fmaf(xv[e], wg[o][e], sg);
          su = fmaf(xv[e], wu[o][e], su);
        }
        acc[r * 8 + o * 2] = sg;
        acc[r * 8 + o * 2 + 1] = su;
      }
    }
  }
  XR<kRG * 8, 32>::run(acc, lane);  // lane l holds index l >> 1 = r*8 + o*2 + {0 gate, 1 up}
  const float other = __shfl_xor(acc[0], 2, 64);
  const int idx = lane >> 1;
  const int r = blockIdx.y * kRG + (idx >> 3), f = f0 + ((idx >> 1) & 3);
  if ((lane & 3) == 0 && r < B && f < F) m[(size_t)r * F + f] = gelu_tanh(acc[0]) * other;
  // logits fill share
  if (fill.logits) {
    const size_t nblk = (size_t)gridDim.x * gridDim.y;
    const size_t bid = (size_t)blockIdx.y * gridDim.x + blockIdx.x;
    const size_t total = fill.end - fill.begin;
    const size_t per = ((total + nblk - 1) / nblk + 3) & ~(size_t)3;
    const size_t a = fill.begin + bid * per;
    const size_t e = a + per < fill.end ? a + per : fill.end;
    if (a < e) {
      const float4 v = make_float4(-1e30f, -1e30f, -1e30f, -1e30f);
      // fill.begin and per are multiples of 4 floats except possibly the range end
      size_t i = a + threadIdx.x * 4;
      for (; i + 4 <= e; i += 1024) *reinterpret_cast<float4*>(fill.logits + i) = v;
      for (; i < e; ++i) fill.logits[i] = -1e30f;
    }
  }
}

// ------------------------------------------------------------------------------------------------------------
// output norm + post_projection + centroid scores ([MTP doc] "Tensor schema": output_norm, assist_post_proj,
// assist_embed_centroids; [Inventory] "Centroid / ordered embeddings LM head", step 1)
// grid ((Bb + C) / 16, ceil(B / 4))

__global__ __launch_bounds__(256) void k_post(int B, int H, int Bb, int C, Residual res,
                                              const uint16_t* __restrict__ w_out, float eps,
                                              const uint16_t* __restrict__ Wp, const uint16_t* __restrict__ Wc,
                                              float* __restrict__ h_out, uint16_t* __restrict__ hidden_out,
                                              float* __restrict__ scores) {
  extern __shared__ float xs[];  // [kRG][H]
  prologue_norm(res, w_out, eps, B, H, xs);
  __syncthreads();
  if (blockIdx.x == 0) {
    for (int i = threadIdx.x; i < kRG * H; i += 256) {
      const int r = blockIdx.y * kRG + i / H;
      if (r < B) h_out[(size_t)r * H + i % H] = xs[i];
    }
  }
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n0 = blockIdx.x * 16 + wave * 4;
  const bool cen = n0 >= Bb;
  float acc[kRG * 4];
  if (!cen)
    wave_dense<4>(xs, H, Wp, H, n0, Bb, acc);
  else
    wave_dense<4>(xs, H, Wc, H, n0 - Bb, C, acc);
  const int idx = lane >> 2;
  const int r = blockIdx.y * kRG + (idx >> 2), n = n0 + (idx & 3);
  if ((lane & 3) == 0 && r < B) {
    if (!cen) {
      if (n < Bb) hidden_out[(size_t)r * Bb + n] = f2bf(acc[0]);
    } else if (n - Bb < C) {
      scores[(size_t)r * C + (n - Bb)] = acc[0];
    }
  }
}

// ------------------------------------------------------------------------------------------------------------
// single-query attention over the shared cache ([MTP doc] "What it is": Q-only attention on the target's
// last-layer K/V; [Guide] section 2(4); [Inventory] "Notes for llama.cpp port" 2: V taken from K)
// grid (nsplit, B * nkv). HD = head_dim, G = query heads per kv head, DPL = dims per lane, KB = keys per batch.

template <int HD, int G>
__global__ __launch_bounds__(256) void k_attn(int B, int nh, int nkv, const float* __restrict__ q,
                                              const uint16_t* __restrict__ qnorm, float eps,
                                              const float* __restrict__ rope, int type, const uint16_t* __restrict__ K,
                                              const uint16_t* __restrict__ Vc, int cap, RowWindows win, int nsplit,
                                              float scale_log2, float* __restrict__ pacc, float* __restrict__ pml,
                                              uint32_t* __restrict__ cnt, float* __restrict__ o) {
  constexpr int DPL = HD / 64;
  constexpr int KB = 64 / G;
  __shared__ float qs[G][HD];
  __shared__ float wml[4][G][2];
  __shared__ float wacc[4][G][HD];
  __shared__ int is_last;
  const int sp = blockIdx.x, bg = blockIdx.y;
  const int b = bg / nkv, g = bg % nkv;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int half = HD / 2;

  // q_norm + rotation at the row's constant position ([Guide] section 2(2))
  const float* tab = rope + ((size_t)b * 2 + type) * 2 * half;
  for (int hh = wave; hh < G; hh += 4) {
    const float* qr = q + ((size_t)b * nh + g * G + hh) * HD;
    float v[DPL];
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) {
      v[e] = qr[lane * DPL + e];
      ss += v[e] * v[e];
    }
    ss = wave_sum(ss);
    const float r = 1.0f / sqrtf(ss / (float)HD + eps);
#pragma unroll
    for (int e = 0; e < DPL; ++e) v[e] = v[e] * r * bf2f(qnorm[lane * DPL + e]);
#pragma unroll
    for (int e = 0; e < DPL; ++e) {
      const float partner = __shfl_xor(v[e], 32, 64);  // dim i <-> i + HD/2
      const int i = (lane & 31) * DPL + e;
      const float c = tab[i], s = tab[half + i];
      qs[hh][lane * DPL + e] = (lane < 32) ? (v[e] * c - partner * s) : (v[e] * c + partner * s);
    }
  }
  __syncthreads();
  float qr[G][DPL];
#pragma unroll
  for (int hh = 0; hh < G; ++hh)
#pragma unroll
    for (int e = 0; e < DPL; ++e) qr[hh][e] = qs[hh][lane * DPL + e];

  const int cntk = win.count[b];
  const int chunk = (cntk + nsplit - 1) / nsplit;
  const int k0 = win.start[b] + sp * chunk;
  const int k1 = min(win.start[b] + cntk, k0 + chunk);
  const bool same_v = (Vc == K);
  const uint16_t* Kb = K + ((size_t)b * nkv + g) * (size_t)cap * HD + lane * DPL;
  const uint16_t* Vb = Vc + ((size_t)b * nkv + g) * (size_t)cap * HD + lane * DPL;

  float mrun[G], lrun[G], acc[G][DPL];
#pragma unroll
  for (int hh = 0; hh < G; ++hh) {
    mrun[hh] = -INFINITY;
    lrun[hh] = 0.f;
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[hh][e] = 0.f;
  }
  const int jl = lane / G, hl = lane % G;

  for (int t0 = k0 + wave * KB; t0 < k1; t0 += 4 * KB) {
    const int nk = min(KB, k1 - t0);
    float kf[KB][DPL];
#pragma unroll
    for (int j = 0; j < KB; ++j) {
      if (j < nk) {
        const uint16_t* p = Kb + (size_t)(t0 + j) * HD;
        if constexpr (DPL == 4) {
          const uint2 w = *reinterpret_cast<const uint2*>(p);
          kf[j][0] = bf_lo(w.x); kf[j][1] = bf_hi(w.x); kf[j][2] = bf_lo(w.y); kf[j][3] = bf_hi(w.y);
        } else if constexpr (DPL == 2) {
          const uint32_t w = *reinterpret_cast<const uint32_t*>(p);
          kf[j][0] = bf_lo(w); kf[j][1] = bf_hi(w);
        } else {
          kf[j][0] = bf2f(p[0]);
        }
      } else {
#pragma unroll
        for (int e = 0; e < DPL; ++e) kf[j][e] = 0.f;
      }
    }
    float sc[64];
#pragma unroll
    for (int j = 0; j < KB; ++j)
#pragma unroll
      for (int hh = 0; hh < G; ++hh) {
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < DPL; ++e) s = fmaf(kf[j][e], qr[hh][e], s);
        sc[j * G + hh] = s;
      }
    XR<64, 32>::run(sc, lane);  // lane l: score of key l / G, head l % G
    float s = (jl < nk) ? sc[0] * scale_log2 : -INFINITY;
    float mx = s;
#pragma unroll
    for (int of = G; of < 64; of <<= 1) mx = fmaxf(mx, __shfl_xor(mx, of, 64));
    float alpha[G];
    float mhl = 0.f;
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      const float mn = fmaxf(mrun[hh], readlane_f(mx, hh));
      alpha[hh] = (mrun[hh] == -INFINITY) ? 0.f : exp2f(mrun[hh] - mn);
      mrun[hh] = mn;
      if (hl == hh) mhl = mn;
    }
    const float p = (jl < nk) ? exp2f(s - mhl) : 0.f;
    float ps = p;
#pragma unroll
    for (int of = G; of < 64; of <<= 1) ps += __shfl_xor(ps, of, 64);
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
      lrun[hh] = lrun[hh] * alpha[hh] + readlane_f(ps, hh);
#pragma unroll
      for (int e = 0; e < DPL; ++e) acc[hh][e] *= alpha[hh];
    }
    // P.V
#pragma unroll
    for (int j = 0; j < KB; ++j) {
      if (j < nk) {
        float vf[DPL];
        if (same_v) {
#pragma unroll
          for (int e = 0; e < DPL; ++e) vf[e] = kf[j][e];
        } else {
          const uint16_t* pv = Vb + (size_t)(t0 + j) * HD;
#pragma unroll
          for (int e = 0; e < DPL; ++e) vf[e] = bf2f(pv[e]);
        }
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
          const float pj = readlane_f(p, j * G + hh);
#pragma unroll
          for (int e = 0; e < DPL; ++e) acc[hh][e] = fmaf(pj, vf[e], acc[hh][e]);
        }
      }
    }
  }
  // combine the 4 waves of this block
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
  for (int i = threadIdx.x; i < G * HD; i += 256) {
    const int hh = i / HD, d = i % HD;
    float M = -INFINITY;
    for (int w = 0; w < 4; ++w) M = fmaxf(M, wml[w][hh][0]);
    float L = 0.f, A = 0.f;
    if (M != -INFINITY) {
      for (int w = 0; w < 4; ++w) {
        if (wml[w][hh][0] == -INFINITY) continue;
        const float f = exp2f(wml[w][hh][0] - M);
        L = fmaf(wml[w][hh][1], f, L);
        A = fmaf(wacc[w][hh][d], f, A);
      }
    }
    const size_t slot = ((size_t)b * nh + g * G + hh) * kMaxSplit + sp;
    pacc[slot * HD + d] = A;
    if (d == 0) {
      pml[slot * 2 + 0] = M;
      pml[slot * 2 + 1] = L;
    }
  }
  // the last block of this (row, kv head) merges all splits
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) is_last = (atomicAdd(&cnt[bg], 1u) == (uint32_t)(nsplit - 1));
  __syncthreads();
  if (!is_last) return;
  __threadfence();
  for (int i = threadIdx.x; i < G * HD; i += 256) {
    const int hh = i / HD, d = i % HD;
    const size_t base = ((size_t)b * nh + g * G + hh) * kMaxSplit;
    float M = -INFINITY;
    for (int s2 = 0; s2 < nsplit; ++s2) M = fmaxf(M, pml[(base + s2) * 2]);
    float L = 0.f, A = 0.f;
    if (M != -INFINITY) {
      for (int s2 = 0; s2 < nsplit; ++s2) {
        const float m2 = pml[(base + s2) * 2];
        if (m2 == -INFINITY) continue;
        const float f = exp2f(m2 - M);
        L = fmaf(pml[(base + s2) * 2 + 1], f, L);
        A = fmaf(pacc[(base + s2) * HD + d], f, A);
      }
    }
    o[((size_t)b * nh + g * G + hh) * HD + d] = (L > 0.f) ? A / L : 0.f;
  }
  if (threadIdx.x == 0) cnt[bg] = 0u;  // every other block of this (row, kv head) has already arrived
}

// ------------------------------------------------------------------------------------------------------------
// masked head ([Inventory] "Centroid / ordered embeddings LM head" steps 2-5)

__global__ __launch_bounds__(256) void k_topk(const float* __restrict__ scores, int C, int k,
                                              int32_t* __restrict__ sel) {
  constexpr int kPer = 32;  // C <= 256 * 32
  __shared__ uint64_t red[4];
  const int b = blockIdx.x;
  uint64_t key[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int c = threadIdx.x + 256 * i;
    key[i] = (c < C) ? (((uint64_t)f32_order(scores[(size_t)b * C + c]) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)c))
                     : 0ull;
  }
  for (int j = 0; j < k; ++j) {
    uint64_t mx = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) mx = u64_max(mx, key[i]);
    mx = block_max_u64(mx, red);
    const uint32_t c = 0xFFFFFFFFu - (uint32_t)(mx & 0xFFFFFFFFull);
    if (threadIdx.x == 0) sel[(size_t)b * k + j] = (int32_t)c;
    if ((int)(c % 256) == (int)threadIdx.x) {
#pragma unroll
      for (int i = 0; i < kPer; ++i)
        if (i == (int)(c / 256)) key[i] = 0ull;
    }
  }
}

// grid (k, B), 256 threads = 16 groups of 16 lanes; each group scores one candidate row at a time.
__global__ __launch_bounds__(256) void k_head(int k, int vsc, int H, const int32_t* __restrict__ sel,
                                              const int32_t* __restrict__ ordering, const uint16_t* __restrict__ E,
                                              const float* __restrict__ h, int32_t* __restrict__ ids,
                                              float* __restrict__ z, float* __restrict__ logits, size_t V,
                                              uint64_t* __restrict__ keys, uint32_t* __restrict__ cnt,
                                              int32_t* __restrict__ next, int32_t* __restrict__ out2, int stride2) {
  extern __shared__ float hs[];  // [H]
  __shared__ uint64_t red[4];
  __shared__ int is_last;
  const int j = blockIdx.x, b = blockIdx.y;
  const int grp = threadIdx.x >> 4, l16 = threadIdx.x & 15;
  for (int i = threadIdx.x; i < H; i += 256) hs[i] = h[(size_t)b * H + i];
  __syncthreads();
  const int c = sel[(size_t)b * k + j];
  uint64_t best = 0;
  for (int t = grp; t < vsc; t += 16) {
    const int id = ordering[(size_t)c * vsc + t];
    const uint16_t* e = E + (size_t)id * H;
    float s = 0.f;
    for (int col = l16 * 8; col < H; col += 128) {
      float ef[8];
      load8(e + col, ef);
#pragma unroll
      for (int q = 0; q < 8; ++q) s = fmaf(ef[q], hs[col + q], s);
    }
#pragma unroll
    for (int of = 8; of > 0; of >>= 1) s += __shfl_xor(s, of, 64);
    if (l16 == 0) {
      const size_t slot = ((size_t)b * k + j) * vsc + t;
      ids[slot] = id;
      z[slot] = s;
      if (logits) logits[(size_t)b * V + id] = s;
      best = u64_max(best, ((uint64_t)f32_order(s) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)id));
    }
  }
  best = block_max_u64(best, red);
  if (threadIdx.x == 0) keys[(size_t)b * k + j] = best;
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) is_last = (atomicAdd(&cnt[b], 1u) == (uint32_t)(k - 1));
  __syncthreads();
  if (!is_last) return;
  __threadfence();
  uint64_t mx = 0;
  for (int i = threadIdx.x; i < k; i += 256) mx = u64_max(mx, keys[(size_t)b * k + i]);
  mx = block_max_u64(mx, red);
  if (threadIdx.x == 0) {
    const int32_t id = (int32_t)(0xFFFFFFFFu - (uint32_t)(mx & 0xFFFFFFFFull));
    next[b] = id;
    if (out2) out2[(size_t)b * stride2] = id;
    cnt[b] = 0u;  // every other block of this row has already arrived
  }
}

__global__ void k_fill(float4* __restrict__ p, size_t n4, float* __restrict__ tail, int ntail) {
  const float4 v = make_float4(-1e30f, -1e30f, -1e30f, -1e30f);
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) p[i] = v;
  if (blockIdx.x == 0 && (int)threadIdx.x < ntail) tail[threadIdx.x] = -1e30f;
}

__global__ void k_zero_u32(uint32_t* __restrict__ p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0u;
}

int row_groups(int B) { return (B + kRG - 1) / kRG; }

}  // namespace

// ------------------------------------------------------------------------------------------------------------
// launchers

hipError_t launch_pre(hipStream_t s, int B, int Bb, int H, int V, const uint16_t* th, const int32_t* tok,
                      const uint16_t* emb, float escale, const uint16_t* w_pre, float* x, uint32_t* counters,
                      int ncounters) {
  dim3 grid((H + 3) / 4, row_groups(B));
  k_pre<<<grid, 256, 0, s>>>(B, Bb, H, V, th, tok, emb, escale, w_pre, x, counters, ncounters);
  return hipGetLastError();
}

hipError_t launch_qproj(hipStream_t s, int B, int H, int QD, Residual res, const uint16_t* w_norm, float eps,
                        const uint16_t* w_q, float* q) {
  dim3 grid((QD + 15) / 16, row_groups(B));
  k_qproj<<<grid, 256, kRG * H * sizeof(float), s>>>(B, H, QD, res, w_norm, eps, w_q, q);
  return hipGetLastError();
}

hipError_t launch_dense(hipStream_t s, int B, int K, int N, const float* X, const uint16_t* w, float* y) {
  dim3 grid((N + 3) / 4, row_groups(B));
  k_dense<<<grid, 256, kRG * K * sizeof(float), s>>>(B, K, N, X, w, y);
  return hipGetLastError();
}

hipError_t launch_ffn(hipStream_t s, int B, int H, int F, Residual res, const uint16_t* w_norm, float eps,
                      const uint16_t* w_gate, const uint16_t* w_up, float* m, FillRange fill) {
  dim3 grid((F + 15) / 16, row_groups(B));
  k_ffn<<<grid, 256, kRG * H * sizeof(float), s>>>(B, H, F, res, w_norm, eps, w_gate, w_up, m, fill);
  return hipGetLastError();
}

hipError_t launch_post(hipStream_t s, int B, int H, int Bb, int C, Residual res, const uint16_t* w_out, float eps,
                       const uint16_t* w_post, const uint16_t* w_cen, float* h_out, uint16_t* hidden_out,
                       float* scores) {
  dim3 grid((Bb + C + 15) / 16, row_groups(B));
  k_post<<<grid, 256, kRG * H * sizeof(float), s>>>(B, H, Bb, C, res, w_out, eps, w_post, w_cen, h_out, hidden_out,
                                                     scores);
  return hipGetLastError();
}

hipError_t launch_attn(hipStream_t s, int B, int nh, int nkv, int hd, const float* q, const uint16_t* qnorm,
                       float eps, const float* rope, int type, const uint16_t* K, const uint16_t* V, int cap,
                       const RowWindows& win, int nsplit, float scale, float* pacc, float* pml, uint32_t* cnt,
                       float* o) {
  dim3 grid(nsplit, B * nkv);
  const float sl2 = scale * 1.4426950408889634f;
  const int G = nh / nkv;
#define MTPD_ATTN(HD_, G_)                                                                                     \
  if (hd == HD_ && G == G_) {                                                                                  \
    k_attn<HD_, G_><<<grid, 256, 0, s>>>(B, nh, nkv, q, qnorm, eps, rope, type, K, V, cap, win, nsplit, sl2, \
                                         pacc, pml, cnt, o);                                                   \
    return hipGetLastError();                                                                                  \
  }
  MTPD_ATTN(256, 1) MTPD_ATTN(256, 2) MTPD_ATTN(256, 4) MTPD_ATTN(256, 8)
  MTPD_ATTN(128, 1) MTPD_ATTN(128, 2) MTPD_ATTN(128, 4) MTPD_ATTN(128, 8)
  MTPD_ATTN(64, 1) MTPD_ATTN(64, 2) MTPD_ATTN(64, 4) MTPD_ATTN(64, 8)
#undef MTPD_ATTN
  return hipErrorInvalidValue;
}

hipError_t launch_topk(hipStream_t s, int B, const float* scores, int C, int k, int32_t* sel) {
  k_topk<<<B, 256, 0, s>>>(scores, C, k, sel);
  return hipGetLastError();
}

hipError_t launch_head(hipStream_t s, int B, int k, int vsc, int H, const int32_t* sel, const int32_t* ordering,
                       const uint16_t* E, const float* h, int32_t* ids, float* z, float* logits, size_t V,
                       uint64_t* keys, uint32_t* cnt, int32_t* next, int32_t* out2, int stride2) {
  dim3 grid(k, B);
  k_head<<<grid, 256, H * sizeof(float), s>>>(k, vsc, H, sel, ordering, E, h, ids, z, logits, V, keys, cnt, next,
                                              out2, stride2);
  return hipGetLastError();
}

hipError_t launch_zero_u32(hipStream_t s, uint32_t* p, int n) {
  k_zero_u32<<<1, 256, 0, s>>>(p, n);
  return hipGetLastError();
}

hipError_t launch_fill(hipStream_t s, float* logits, size_t n) {
  const size_t n4 = n / 4;
  const int ntail = (int)(n - n4 * 4);
  size_t grid = (n4 + 255) / 256;
  if (grid > 4096) grid = 4096;
  if (grid < 1) grid = 1;
  k_fill<<<(unsigned)grid, 256, 0, s>>>(reinterpret_cast<float4*>(logits), n4, logits + n4 * 4, ntail);
  return hipGetLastError();
}

}  // namespace mtpd
