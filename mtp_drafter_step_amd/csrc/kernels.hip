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
// Latency rules followed throughout (every stage of a drafter step is latency-bound except the long attention and
// the head gather): loads are issued unconditionally from clamped addresses and masked afterwards, with trip counts
// that the compiler can see are wave-uniform, so that a wave keeps all its loads in flight at once; weights that do
// not depend on the previous stage are requested before the block waits on that stage's activations; no block
// waits on another block inside a launch.
//
// Dense kernels: a block owns a tile of outputs for a group of 4 batch rows; each wave computes a few outputs for
// the 4 rows with lanes striding the reduction dimension (4 elements per lane per 256-wide chunk), then a butterfly
// transpose-reduction leaves one finished (row, output) sum per lane group.
#include "kernels.h"

#include <hip/hip_ext.h>

#include <math.h>
#include <stdlib.h>

#include <type_traits>

namespace mtpd {

namespace {

constexpr int kRG = kRowGroup;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }
__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// fp32 -> bf16, round to nearest even (finite inputs)
__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}


// order-preserving map of fp32 onto uint32 (larger float -> larger integer)
__device__ __forceinline__ uint32_t f32_order(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// (value, id) key: larger value first, then lower id
__device__ __forceinline__ uint64_t vid_key(float v, uint32_t id) {
  return ((uint64_t)f32_order(v) << 32) | (uint64_t)(0xFFFFFFFFu - id);
}
__device__ __forceinline__ int32_t key_id(uint64_t k) { return (int32_t)(0xFFFFFFFFu - (uint32_t)(k & 0xFFFFFFFFull)); }

__device__ __forceinline__ uint64_t u64_max(uint64_t a, uint64_t b) { return a > b ? a : b; }

// 16-byte load through the global address space: a generic (flat) load would also count against the LDS wait
// counter, so a wait for LDS reads would drain the outstanding memory loads too
__device__ __forceinline__ uint4 ld_global16(const void* p) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  return __builtin_bit_cast(uint4, *(const __attribute__((address_space(1))) u32x4*)(p));
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)v, o, 64);
    const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), o, 64);
    v = u64_max(v, ((uint64_t)hi << 32) | lo);
  }
  return v;
}

__device__ __forceinline__ float gelu_tanh(float a) {
  const float c = 0.7978845608028654f;  // sqrt(2/pi)
  return 0.5f * a * (1.0f + tanhf(c * (a + 0.044715f * a * a * a)));
}

__device__ __forceinline__ float readlane_f(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// Butterfly transpose-reduction of V per-lane values over lanes differing in bits O, O/2, ..., 1. Afterwards v[0]
// of lane l holds the sum over those lanes of the value whose index is given by the lane bits consumed by the
// halving steps (the highest bit first).
//
// The exchanges stay in the vector ALU: lanes 32 apart and 16 apart swap through v_permlane32_swap /
// v_permlane16_swap applied to the value pair itself (the swap leaves each lane its own kept value and its
// partner's, so one add finishes the step); within rows of 16 lanes DPP moves supply the partner: a rotation by 8
// (the partner 8 away), the half-row mirror (lane i <-> 7 - i: opposite bit 2, and the two later steps over bits 1
// and 0 still cover all eight lanes), and quad permutations for bits 1 and 0.
template <int O>
__device__ __forceinline__ float xr_partner(float v) {
  const int x = __float_as_int(v);
  if constexpr (O == 8) return __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0x128, 0xf, 0xf, false));  // row_ror:8
  if constexpr (O == 4) return __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0x141, 0xf, 0xf, false));  // half mirror
  if constexpr (O == 2) return __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0x4E, 0xf, 0xf, false));   // [2,3,0,1]
  if constexpr (O == 1) return __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0xB1, 0xf, 0xf, false));   // [1,0,3,2]
  if constexpr (O == 32 || O == 16) {
    // swapping a value with itself leaves each lane its own value and its partner's, in the slot set by the lane
    // bit O
    const unsigned u = __float_as_uint(v);
    if constexpr (O == 32) {
      const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
      return __uint_as_float((__lane_id() & 32) ? r[0] : r[1]);
    } else {
      const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
      return __uint_as_float((__lane_id() & 16) ? r[0] : r[1]);
    }
  }
  return v;
}

// (lo, hi) pair step over lanes O apart for O = 32 / 16: returns, per lane, the kept value plus the partner's
template <int O>
__device__ __forceinline__ float xr_swap_sum(float lo, float hi) {
  const unsigned a = __float_as_uint(lo), c = __float_as_uint(hi);
  if constexpr (O == 32) {
    const auto r = __builtin_amdgcn_permlane32_swap(a, c, false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  } else {
    const auto r = __builtin_amdgcn_permlane16_swap(a, c, false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
  }
}

template <int V, int O>
struct XR {
  static __device__ __forceinline__ void run(float* v, int lane) {
    if constexpr (V > 1) {
      constexpr int H = V / 2;
      if constexpr (O == 32 || O == 16) {
#pragma unroll
        for (int i = 0; i < H; ++i) v[i] = xr_swap_sum<O>(v[i], v[i + H]);
      } else {
        const bool up = (lane & O) != 0;
#pragma unroll
        for (int i = 0; i < H; ++i) {
          const float send = up ? v[i] : v[i + H];
          const float keep = up ? v[i + H] : v[i];
          v[i] = keep + xr_partner<O>(send);
        }
      }
      if constexpr (O > 1) XR<H, O / 2>::run(v, lane);
    } else {
      if constexpr (O == 32 || O == 16)
        v[0] = xr_swap_sum<O>(v[0], v[0]);
      else
        v[0] += xr_partner<O>(v[0]);
      if constexpr (O > 1) XR<1, O / 2>::run(v, lane);
    }
  }
};

// Sum over the wave, left in every lane (the exchanges of XR, with nothing to transpose).
__device__ __forceinline__ float wave_sum(float v) {
  XR<1, 32>::run(&v, 0);
  return v;
}

__device__ __forceinline__ void unpack4(uint2 w, float* f) {
  f[0] = bf_lo(w.x); f[1] = bf_hi(w.x); f[2] = bf_lo(w.y); f[3] = bf_hi(w.y);
}
__device__ __forceinline__ void unpack8(uint4 w, float* f) {
  f[0] = bf_lo(w.x); f[1] = bf_hi(w.x); f[2] = bf_lo(w.y); f[3] = bf_hi(w.y);
  f[4] = bf_lo(w.z); f[5] = bf_hi(w.z); f[6] = bf_lo(w.w); f[7] = bf_hi(w.w);
}

// ------------------------------------------------------------------------------------------------------------
// dense building blocks
//
// Every trip count below is a template parameter, and every load a wave needs is issued before any loaded value is
// used: a load inside a data-dependent branch, or inside a loop whose bound the compiler cannot see, is followed by
// its own wait, which turns one memory round trip into one per element.

// Weights of OPW consecutive output rows for one wave: IT chunks of 256 along K, 4 bf16 per lane per chunk.
template <int OPW, int IT>
struct WaveW {
  uint2 w[OPW][IT];
  __device__ __forceinline__ void load(const uint16_t* W, int K, int n0, int N) {
    const int lane = lane_id();
#pragma unroll
    for (int o = 0; o < OPW; ++o) {
      const uint16_t* row = W + (size_t)min(n0 + o, N - 1) * K + lane * 4;
#pragma unroll
      for (int i = 0; i < IT; ++i) w[o][i] = *reinterpret_cast<const uint2*>(row + i * 256);
    }
  }
  // acc[r*OPW + o] = sum_k X(r, k) W[n0+o][k] for the kRG rows at xrow[r] (fp32, LDS or global); afterwards lane l
  // holds the finished sum of (row, output) index l >> (6 - log2(kRG*OPW)) in acc[0] (transpose-reduction).
  __device__ __forceinline__ void dot(const float* const* xrow, float* acc) const {
    const int lane = lane_id();
    float4 xr[kRG][IT];
#pragma unroll
    for (int r = 0; r < kRG; ++r)
#pragma unroll
      for (int i = 0; i < IT; ++i) xr[r][i] = *reinterpret_cast<const float4*>(xrow[r] + i * 256 + lane * 4);
#pragma unroll
    for (int i = 0; i < kRG * OPW; ++i) acc[i] = 0.f;
#pragma unroll
    for (int i = 0; i < IT; ++i)
#pragma unroll
      for (int o = 0; o < OPW; ++o) {
        float wf[4];
        unpack4(w[o][i], wf);
#pragma unroll
        for (int r = 0; r < kRG; ++r) {
          float s = acc[r * OPW + o];
          s = fmaf(xr[r][i].x, wf[0], s);
          s = fmaf(xr[r][i].y, wf[1], s);
          s = fmaf(xr[r][i].z, wf[2], s);
          s = fmaf(xr[r][i].w, wf[3], s);
          acc[r * OPW + o] = s;
        }
      }
    XR<kRG * OPW, 32>::run(acc, lane);
  }
};

// Residual update + RMSNorm for the block's row group into LDS xs[kRG][H] (H = 64 NPL); one wave per row. Rows
// beyond B are zero. Block column 0 stores x_new when res.x_new is set. The delta is the sum of res.nd <= ND
// partials (ND a power of two; the surplus loads are clamped to the last partial and weighted by zero).
// Branch-free: the delta loads are always issued (from x_old when there is no delta) and their effect selected
// afterwards.
template <int NPL, int ND>
__device__ __forceinline__ void prologue_norm(const Residual& res, const uint16_t* w_norm, float eps, int B,
                                              float* xs) {
  constexpr int H = NPL * 64;
  const int wave = wave_id(), lane = lane_id();
  const int row = blockIdx.y * kRG + wave;
  const int rr = min(row, B - 1);
  const bool hasd = res.delta != nullptr;
  const float* xo = res.x_old + (size_t)rr * H;
  const float* dr = hasd ? res.delta + (size_t)rr * H : xo;
  const size_t dst = hasd ? res.dstride : 0;
  const int nd = hasd ? res.nd : 1;
  const uint16_t* wdp = hasd ? res.w_delta : w_norm;
  float xv[NPL], dp[ND][NPL];
  uint16_t wv[NPL], wd[NPL];
#pragma unroll
  for (int j = 0; j < NPL; ++j) {
    xv[j] = xo[lane + 64 * j];
    wv[j] = w_norm[lane + 64 * j];
    wd[j] = wdp[lane + 64 * j];
  }
#pragma unroll
  for (int p = 0; p < ND; ++p)
#pragma unroll
    for (int j = 0; j < NPL; ++j) dp[p][j] = dr[(size_t)min(p, nd - 1) * dst + lane + 64 * j];
  float dv[NPL];
#pragma unroll
  for (int j = 0; j < NPL; ++j) {
    float a = dp[0][j];
#pragma unroll
    for (int p = 1; p < ND; ++p) a += (p < nd) ? dp[p][j] : 0.f;
    dv[j] = a;
  }
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < NPL; ++j) ss = fmaf(dv[j], dv[j], ss);
  ss = wave_sum(ss);
  const float r = 1.0f / sqrtf(ss / (float)H + eps);
#pragma unroll
  for (int j = 0; j < NPL; ++j) xv[j] = hasd ? (xv[j] + dv[j] * r * bf2f(wd[j])) * res.scale : xv[j];
  float s2 = 0.f;
#pragma unroll
  for (int j = 0; j < NPL; ++j) s2 = fmaf(xv[j], xv[j], s2);
  s2 = wave_sum(s2);
  const float r2 = 1.0f / sqrtf(s2 / (float)H + eps);
  const bool valid = row < B;
  if (res.x_new && blockIdx.x == 0 && valid) {
#pragma unroll
    for (int j = 0; j < NPL; ++j) res.x_new[(size_t)row * H + lane + 64 * j] = xv[j];
  }
  float* xr = xs + wave * H;
#pragma unroll
  for (int j = 0; j < NPL; ++j) xr[lane + 64 * j] = valid ? xv[j] * r2 * bf2f(wv[j]) : 0.f;
}

// ------------------------------------------------------------------------------------------------------------
// pre_projection of [target hidden ; embedded token]  ([MTP doc] "What it is": 2x backbone input;
// [Guide] section 2(3)). grid (ceil(H / 4), ceil(B / 4)), NWV waves. A block computes 4 outputs for 4 rows; its waves
// split K = 2 Bb into 256-wide chunks (CPW per wave; a chunk lies wholly in the hidden half or the embedding half,
// since Bb % 256 == 0), and the partial sums meet in LDS. Weight and hidden loads are issued before the token is
// known; the embedding rows right after.

template <int NWV, int CPW>
__global__ __launch_bounds__(NWV * 64) void k_pre(int B, int Bb, int H, int V, const uint16_t* __restrict__ th,
                                                  TokenSource ts, const uint16_t* __restrict__ emb, float escale,
                                                  const uint16_t* __restrict__ W, float* __restrict__ x) {
  __shared__ int tok_s[kRG];
  __shared__ float red[NWV][16];
  const int wave = wave_id(), lane = lane_id();
  const int r0 = blockIdx.y * kRG;
  const int n0 = blockIdx.x * 4;
  const int K = 2 * Bb;
  const int nch = K >> 8, hch = Bb >> 8;  // chunks in total / in the hidden half
  // the token source of row r0 + wave is requested first (waves beyond kRG repeat row r0), then the weights and
  // hidden-half activations, which do not depend on it
  const int bt = min(r0 + min(wave, kRG - 1), B - 1);
  const uint64_t kraw = ts.keys[(size_t)bt * ts.k + min(lane, ts.k - 1)];
  const int traw = ts.tok[bt];
  __builtin_amdgcn_sched_barrier(0);  // keep these loads ahead of the weight loads (waits count in issue order)
  uint2 wr[CPW][4], xr[CPW][kRG];
  int cidx[CPW];
#pragma unroll
  for (int c = 0; c < CPW; ++c) {
    cidx[c] = min(wave * CPW + c, nch - 1);
    const int k = cidx[c] * 256 + lane * 4;
#pragma unroll
    for (int o = 0; o < 4; ++o) wr[c][o] = *reinterpret_cast<const uint2*>(W + (size_t)min(n0 + o, H - 1) * K + k);
#pragma unroll
    for (int r = 0; r < kRG; ++r)
      xr[c][r] = *reinterpret_cast<const uint2*>(th + (size_t)min(r0 + r, B - 1) * Bb + min(k, Bb - 4));
  }
  if (wave < kRG) {
    int t = traw;
    if (ts.use_keys) {
      t = key_id(wave_max_u64(lane < ts.k ? kraw : 0ull));
      if (blockIdx.x == 0 && lane == 0 && r0 + wave < B) {
        if (ts.out) ts.out[(size_t)bt * ts.out_stride] = t;
        if (ts.next) ts.next[bt] = t;
      }
    }
    t = t < 0 ? 0 : (t >= V ? V - 1 : t);  // out-of-range ids are clamped (documented in the ABI)
    if (lane == 0) tok_s[wave] = t;
  }
  __syncthreads();
  // embedding-half activations (chunks of the hidden half keep their hidden values)
#pragma unroll
  for (int c = 0; c < CPW; ++c) {
    const int k = cidx[c] * 256 + lane * 4;
#pragma unroll
    for (int r = 0; r < kRG; ++r) {
      const uint2 e = *reinterpret_cast<const uint2*>(emb + (size_t)tok_s[r] * Bb + max(k - Bb, 0));
      xr[c][r] = (cidx[c] >= hch) ? e : xr[c][r];
    }
  }
  float acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
  for (int c = 0; c < CPW; ++c) {
    const bool live = wave * CPW + c < nch;
    const float sc = live ? (cidx[c] >= hch ? escale : 1.0f) : 0.0f;
#pragma unroll
    for (int r = 0; r < kRG; ++r) {
      float xf[4];
      unpack4(xr[c][r], xf);
#pragma unroll
      for (int e = 0; e < 4; ++e) xf[e] *= sc;
#pragma unroll
      for (int o = 0; o < 4; ++o) {
        float wf[4];
        unpack4(wr[c][o], wf);
        float s = acc[r * 4 + o];
#pragma unroll
        for (int e = 0; e < 4; ++e) s = fmaf(xf[e], wf[e], s);
        acc[r * 4 + o] = s;
      }
    }
  }
  XR<16, 32>::run(acc, lane);  // lanes 4i .. 4i+3 hold the wave's partial of (row, output) index i
  if ((lane & 3) == 0) red[wave][lane >> 2] = acc[0];
  __syncthreads();
  if (threadIdx.x < 16) {
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < NWV; ++w) s += red[w][threadIdx.x];
    const int r = r0 + (threadIdx.x >> 2), n = n0 + (threadIdx.x & 3);
    if (r < B && n < H) x[(size_t)r * H + n] = s;
  }
}

// ------------------------------------------------------------------------------------------------------------
// q projection ([MTP doc] "Tensor schema": attn_norm, attn_q); grid (QD / 16, ceil(B / 4)), H = 64 NPL

template <int NPL>
__global__ __launch_bounds__(256) void k_qproj(int B, int QD, Residual res, const uint16_t* __restrict__ w_norm,
                                               float eps, const uint16_t* __restrict__ W, float* __restrict__ q) {
  constexpr int H = NPL * 64;
  __shared__ __attribute__((aligned(16))) float xs[kRG][H];
  const int wave = wave_id(), lane = lane_id();
  const int n0 = blockIdx.x * 16 + wave * 4;
  WaveW<4, H / 256> ww;
  ww.load(W, H, n0, QD);
  prologue_norm<NPL, 1>(res, w_norm, eps, B, &xs[0][0]);
  __syncthreads();
  const float* xrow[kRG] = {xs[0], xs[1], xs[2], xs[3]};
  float acc[kRG * 4];
  ww.dot(xrow, acc);
  const int idx = lane >> 2;  // r * 4 + o
  const int r = blockIdx.y * kRG + (idx >> 2), n = n0 + (idx & 3);
  if ((lane & 3) == 0 && r < B && n < QD) q[(size_t)r * QD + n] = acc[0];
}

// ------------------------------------------------------------------------------------------------------------
// Dense product for o_proj / down / centroid scores: grid (N / 4, ceil(B / 4)), K = 256 IT; X rows read directly
// (rows beyond B read row B-1, results discarded).

template <int IT>
__global__ __launch_bounds__(256) void k_dense(int B, int N, const float* __restrict__ X,
                                               const uint16_t* __restrict__ W, float* __restrict__ y) {
  constexpr int K = IT * 256;
  const int wave = wave_id(), lane = lane_id();
  const int n = blockIdx.x * 4 + wave;
  const int r0 = blockIdx.y * kRG;
  WaveW<1, IT> ww;
  ww.load(W, K, n, N);
  const float* xrow[kRG];
#pragma unroll
  for (int r = 0; r < kRG; ++r) xrow[r] = X + (size_t)min(r0 + r, B - 1) * K;
  float acc[kRG];
  ww.dot(xrow, acc);
  const int idx = lane >> 4;
  if ((lane & 15) == 0 && r0 + idx < B && n < N) y[(size_t)(r0 + idx) * N + n] = acc[0];
}

// ------------------------------------------------------------------------------------------------------------
// GeGLU FFN input half ([MTP doc] "Tensor schema": ffn_norm, ffn_gate, ffn_up): grid (F / 16, ceil(B / 4)).
// Each wave: 4 ffn indices x {gate, up} for the 4 rows. Blocks also fill their share of the logits row.

template <int NPL, int ND>
__global__ __launch_bounds__(256) void k_ffn(int B, int F, Residual res, const uint16_t* __restrict__ w_norm,
                                             float eps, const uint16_t* __restrict__ Wg,
                                             const uint16_t* __restrict__ Wu, float* __restrict__ m,
                                             FillRange fill) {
  constexpr int H = NPL * 64;
  __shared__ __attribute__((aligned(16))) float xs[kRG][H];
  const int wave = wave_id(), lane = lane_id();
  const int f0 = blockIdx.x * 16 + wave * 4;
  WaveW<4, H / 256> wg, wu;
  wg.load(Wg, H, f0, F);
  wu.load(Wu, H, f0, F);
  prologue_norm<NPL, ND>(res, w_norm, eps, B, &xs[0][0]);
  __syncthreads();
  const float* xrow[kRG] = {xs[0], xs[1], xs[2], xs[3]};
  float ag[kRG * 4], au[kRG * 4];
  wg.dot(xrow, ag);
  wu.dot(xrow, au);
  const int idx = lane >> 2;
  const int r = blockIdx.y * kRG + (idx >> 2), f = f0 + (idx & 3);
  if ((lane & 3) == 0 && r < B && f < F) m[(size_t)r * F + f] = gelu_tanh(ag[0]) * au[0];
  // logits fill share ([Inventory] "Centroid / ordered embeddings LM head", step 5: the -1e30 base row)
  if (fill.logits) {
    const size_t nblk = (size_t)gridDim.x * gridDim.y;
    const size_t bid = (size_t)blockIdx.y * gridDim.x + blockIdx.x;
    const size_t total = fill.end - fill.begin;
    const size_t per = ((total + nblk - 1) / nblk + 3) & ~(size_t)3;
    const size_t a = fill.begin + bid * per;
    const size_t e = a + per < fill.end ? a + per : fill.end;
    if (a < e) {  // streaming stores: the row is not read again in this kernel or the next
      const f32x4 v = f32x4{-1e30f, -1e30f, -1e30f, -1e30f};
      size_t i = a + threadIdx.x * 4;
      for (; i + 4 <= e; i += 1024) __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(fill.logits + i));
      for (; i < e; ++i) __builtin_nontemporal_store(-1e30f, fill.logits + i);
    }
  }
}

// ------------------------------------------------------------------------------------------------------------
// output norm + post_projection + centroid scores ([MTP doc] "Tensor schema": output_norm, assist_post_proj,
// assist_embed_centroids; [Inventory] "Centroid / ordered embeddings LM head", step 1)
// grid ((Bb + C) / 32, ceil(B / 4)); each wave computes 8 outputs for the 4 rows

template <int NPL>
__global__ __launch_bounds__(256) void k_post(int B, int Bb, int C, Residual res, const uint16_t* __restrict__ w_out,
                                              float eps, const uint16_t* __restrict__ Wp,
                                              const uint16_t* __restrict__ Wc, float* __restrict__ h_out,
                                              uint16_t* __restrict__ hidden_out, float* __restrict__ scores,
                                              uint64_t* __restrict__ keys_zero) {
  constexpr int H = NPL * 64;
  __shared__ __attribute__((aligned(16))) float xs[kRG][H];
  const int wave = wave_id(), lane = lane_id();
  const int n0 = blockIdx.x * 32 + wave * 8;
  const bool cen = n0 >= Bb;  // Bb % 32 == 0: a block is wholly post_proj or wholly centroids
  WaveW<8, H / 256> ww;
  ww.load(cen ? Wc : Wp, H, cen ? n0 - Bb : n0, cen ? C : Bb);
  prologue_norm<NPL, 1>(res, w_out, eps, B, &xs[0][0]);
  __syncthreads();
  if (blockIdx.x == 0) {
    for (int i = threadIdx.x; i < kRG * H; i += 256) {
      const int r = blockIdx.y * kRG + i / H;
      if (r < B) h_out[(size_t)r * H + i % H] = xs[0][i];
    }
    // the dense head accumulates its argmax keys by atomic max from zero
    if (keys_zero && threadIdx.x < kRG && blockIdx.y * kRG + threadIdx.x < B) keys_zero[blockIdx.y * kRG + threadIdx.x] = 0ull;
  }
  const float* xrow[kRG] = {xs[0], xs[1], xs[2], xs[3]};
  float acc[kRG * 8];
  ww.dot(xrow, acc);
  const int idx = lane >> 1;  // r * 8 + o
  const int r = blockIdx.y * kRG + (idx >> 3), n = n0 + (idx & 7);
  if ((lane & 1) == 0 && r < B) {
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
  const uint16_t* Kb = K + ((size_t)b * nkv + g) * (size_t)cap * HD + lane * DPL;
  const uint16_t* Vb = Vc + ((size_t)b * nkv + g) * (size_t)cap * HD + lane * DPL;
  // first batch of keys in flight before the q prologue
  Raw kcur[KB], knext[KB];
  int t0 = k0 + wave * KB;
  if (t0 < k1) {
#pragma unroll
    for (int j = 0; j < KB; ++j) kcur[j] = *reinterpret_cast<const Raw*>(Kb + (size_t)min(t0 + j, k1 - 1) * HD);
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
    const float r = 1.0f / sqrtf(ss / (float)HD + eps);
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
      for (int j = 0; j < KB; ++j) knext[j] = *reinterpret_cast<const Raw*>(Kb + (size_t)min(tn + j, k1 - 1) * HD);
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
      alpha[hh] = (mrun[hh] == -INFINITY) ? 0.f : exp2f(mrun[hh] - mn);
      mrun[hh] = mn;
      mhl = (hl == hh) ? mn : mhl;
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
    // P.V (p of masked keys is 0)
    Raw vraw[KB];
    if (!same_v) {
#pragma unroll
      for (int j = 0; j < KB; ++j) vraw[j] = *reinterpret_cast<const Raw*>(Vb + (size_t)min(t0 + j, k1 - 1) * HD);
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
        const float f = (mw == -INFINITY) ? 0.f : exp2f(mw - M);
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

// Matrix-core variant for head_dim 256 and up to 8 query heads per kv head (heads padded to the 16 rows of an
// MFMA tile). Per wave and batch of 16 keys:
//   S[16 keys][16 heads] = K_tile . q^T with v_mfma_f32_16x16x32_bf16: the key rows load straight into the A
//     operand (lane l: key l%16, 8 dims at 8*(l/16) of each 32-dim step); the fp32 query is split into two bf16
//     terms q = q_hi + q_lo (relative error <= 2^-16) so the product keeps fp32-level accuracy;
//   online softmax on the S layout (lane l holds keys 4*(l/16)+r of head l%16);
//   O[16 heads][256] += P . V with v_mfma_f32_16x16x16_bf16: P (split into bf16 hi + lo) is already in the A layout,
//     V comes from the wave's LDS copy of the key tile read column-wise (4 keys of one dim per lane).


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
  __shared__ __attribute__((aligned(16))) uint16_t qop[KSTEPS][2][G][4][8];  // [step][hi/lo][head][kq][8 dims]
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
  const uint16_t* Kb = K + ((size_t)b * nkv + g) * (size_t)cap * HD + 8 * kq;
  const uint16_t* Vb = Vc + ((size_t)b * nkv + g) * (size_t)cap * HD + 8 * kq;

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
    const uint16_t* r = Kb + (size_t)min(t0 + hq, k1 - 1) * HD;
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
    const float r = 1.0f / sqrtf(ss / (float)HD + eps);
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
  for (int i = threadIdx.x; i < KSTEPS * G * 4 * 8; i += NW * 64) {
    const int e = i & 7, kk = (i >> 3) & 3, hh = (i >> 5) % G, c = i / (32 * G);
    const float v = qs[hh][32 * c + 8 * kk + e];
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
  const int hsel = hq < G ? hq : 0;

  for (; t0 < k1; t0 += S) {
    const int tb = t0;
    {
      const uint16_t* r = Kb + (size_t)min(t0 + S + hq, k1 - 1) * HD;
#pragma unroll
      for (int c = 0; c < KSTEPS; ++c) kn[c] = *reinterpret_cast<const uint4*>(r + 32 * c);
    }
    const int nk = min(16, k1 - tb);
    // V tile into this wave's LDS (row = key hq, dims 32c + 8kq .. +8)
    if (same_v) {
#pragma unroll
      for (int c = 0; c < KSTEPS; ++c) *reinterpret_cast<uint4*>(tile + hq * LROW + 32 * c + 8 * kq) = ka[c];
    } else {
      const uint16_t* r = Vb + (size_t)min(tb + hq, k1 - 1) * HD;
#pragma unroll
      for (int c = 0; c < KSTEPS; ++c)
        *reinterpret_cast<uint4*>(tile + hq * LROW + 32 * c + 8 * kq) = *reinterpret_cast<const uint4*>(r + 32 * c);
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
    const float alpha = (mrun == -INFINITY) ? 0.f : exp2f(mrun - mn);
    float pv[4], ps = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      pv[r] = (sv[r] == -INFINITY) ? 0.f : exp2f(sv[r] - mn);
      ps += pv[r];
    }
    ps += xr_partner<16>(ps);
    ps += xr_partner<32>(ps);
    lrun = lrun * alpha + ps;
    mrun = mn;
    i16x4 phi, plo;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint16_t hb = f2bf(pv[r]);
      phi[r] = (short)hb;
      plo[r] = (short)f2bf(pv[r] - bf2f(hb));
    }
    // rescale the accumulators: D rows are heads 4kq + r, whose alpha lives in lane 4kq + r (rows of heads >= G
    // are padding)
    float al[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      al[r] = readlane_f(alpha, r);
      if constexpr (GQ > 1) al[r] = (kq == 1) ? readlane_f(alpha, 4 + r) : al[r];
    }
#pragma unroll
    for (int t = 0; t < TILES; ++t) {
      i16x4 vb;
#pragma unroll
      for (int r = 0; r < 4; ++r) vb[r] = (short)tile[(4 * kq + r) * LROW + 16 * t + hq];
      f32x4 a = acc[t];
#pragma unroll
      for (int r = 0; r < 4; ++r) a[r] *= al[r];
      a = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(phi, vb, a, 0, 0, 0);
      a = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(plo, vb, a, 0, 0, 0);
      acc[t] = a;
    }
#pragma unroll
    for (int c = 0; c < KSTEPS; ++c) ka[c] = kn[c];
  }
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
        const float f = (mw == -INFINITY) ? 0.f : exp2f(mw - M);
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

// o_proj partial of chunk c = blockIdx.y of the attention output (dims [256c, 256c + 256)) for row b = blockIdx.z:
// thread i first forms o[b][256c + i], either read directly (NS == 1: the attention wrote o) or merged from the
// nsplit <= NS key-range partials of its head (log-sum-exp weights; the NS loads are issued unconditionally from
// clamped slots and the surplus weighted by zero); then wave w computes outputs 64 bx + 16 w .. +16 over the chunk
// ([MTP doc] "Tensor schema": attn_output). grid (ceil(N / 64), QD / 256, B), 256 threads. (No restrict on the
// loaded arrays: it would let their loads sink below the issue barrier.)
template <int NS>
__global__ __launch_bounds__(256) void k_oproj(int N, int QD, int hd, int nh, int nsplit, const float* o,
                                               const float* pacc, const float* pml, const uint16_t* W,
                                               float* __restrict__ t) {
  static_assert(NS >= 1 && NS <= 64, "one (max, sum) pair per lane");
  __shared__ __attribute__((aligned(16))) float os[256];
  const int wave = wave_id(), lane = lane_id();
  const int c = blockIdx.y, b = blockIdx.z;
  const int n0 = blockIdx.x * 64 + wave * 16;
  const int k0 = c * 256;
  uint2 w[16];
#pragma unroll
  for (int q = 0; q < 16; ++q) w[q] = *reinterpret_cast<const uint2*>(W + (size_t)min(n0 + q, N - 1) * QD + k0 + lane * 4);
  const int d = k0 + (int)threadIdx.x;
  const int h = d / hd, dh = d - h * hd;
  float val;
  if constexpr (NS == 1) {
    val = o[(size_t)b * QD + d];
  } else {
    // a wave's 64 dims lie in one head (head_dim is a multiple of 64): lane s reads split s's (max, sum) pair,
    // the wave forms the merge weights, and each thread takes them by lane index
    const size_t base = ((size_t)b * nh + h) * kMaxSplit;
    float a[NS];
#pragma unroll
    for (int s2 = 0; s2 < NS; ++s2) a[s2] = pacc[(base + (size_t)min(s2, nsplit - 1)) * hd + dh];
    const float2 ml = *reinterpret_cast<const float2*>(pml + (base + (size_t)min(lane, nsplit - 1)) * 2);
    asm volatile("" ::: "memory");  // every load above issued before the first wait
    __builtin_amdgcn_sched_barrier(0);
    const float mv = lane < nsplit ? ml.x : -INFINITY;
    float M = mv;
    M = fmaxf(M, xr_partner<32>(M));
    M = fmaxf(M, xr_partner<16>(M));
    M = fmaxf(M, xr_partner<8>(M));
    M = fmaxf(M, xr_partner<4>(M));
    M = fmaxf(M, xr_partner<2>(M));
    M = fmaxf(M, xr_partner<1>(M));
    const float f = (mv == -INFINITY) ? 0.f : exp2f(mv - M);
    const float L = wave_sum(ml.y * f);
    float A = 0.f;
#pragma unroll
    for (int s2 = 0; s2 < NS; ++s2) A = fmaf(a[s2], readlane_f(f, s2), A);
    val = (L > 0.f) ? A / L : 0.f;
  }
  os[threadIdx.x] = val;
  __syncthreads();
  const float4 xv = *reinterpret_cast<const float4*>(os + lane * 4);
  float acc[16];
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    float wf[4];
    unpack4(w[q], wf);
    acc[q] = fmaf(xv.x, wf[0], fmaf(xv.y, wf[1], fmaf(xv.z, wf[2], xv.w * wf[3])));
  }
  XR<16, 32>::run(acc, lane);  // lane l holds output l >> 2 of the wave's 16
  const int n = n0 + (lane >> 2);
  if ((lane & 3) == 0 && n < N) t[((size_t)c * gridDim.z + b) * N + n] = acc[0];
}

// ------------------------------------------------------------------------------------------------------------
// masked head ([Inventory] "Centroid / ordered embeddings LM head" steps 2-5)
// grid (k, B), 256 threads. Every block of a row recomputes the row's top-k (radix select over order-preserving
// keys; exact, ties to the lower index) and keeps its slot j; 16 groups of 16 lanes then score the slot's cluster.

// NPT scores per thread (C <= 256 NPT), H = 128 HCH. Every score and hidden-state load is issued before the first
// wait. Es is the head table in cluster order (row r = token_embd[ordering[r]]), so the selected cluster's rows are
// contiguous and load together with their token ids. (No restrict on the loaded arrays: it would let the loads
// sink below the issue barriers.)
template <int NPT, int HCH>
__global__ __launch_bounds__(256) void k_head(int C, int k, int vsc, const float* scores, const int32_t* ordering,
                                              const uint16_t* Es, const float* h, int32_t* __restrict__ sel,
                                              int32_t* __restrict__ ids, float* __restrict__ z,
                                              float* __restrict__ logits, size_t V, uint64_t* __restrict__ keys) {
  constexpr int H = HCH * 128;
  constexpr int HPT = (H + 255) / 256;  // hidden elements per thread
  __shared__ uint32_t hist[2][4][256];  // per wave (fewer same-address atomics), double-buffered
  __shared__ uint32_t sh_digit, sh_before, sh_n;
  __shared__ uint64_t cand[kMaxCentroids];
  __shared__ int sh_c;
  __shared__ float hs[H];
  __shared__ uint64_t red[4];
  const int j = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();

  float sv[NPT], hv[HPT];
#pragma unroll
  for (int i = 0; i < NPT; ++i) sv[i] = scores[(size_t)b * C + min(tid + 256 * i, C - 1)];
#pragma unroll
  for (int i = 0; i < HPT; ++i) hv[i] = h[(size_t)b * H + min(tid + 256 * i, H - 1)];
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < HPT; ++i)
    if (tid + 256 * i < H) hs[tid + 256 * i] = hv[i];
  // scores -> order keys; entries beyond C never take part
  uint32_t ok[NPT];
#pragma unroll
  for (int i = 0; i < NPT; ++i) ok[i] = f32_order(sv[i]);

  // Slot j holds the (j+1)-th element in descending (score, then ascending index) order. Radix select on the order
  // keys, 8 bits at a time from the top, narrows the search to the digit bin that holds that rank; once the bin
  // holds a single element, that element is the answer. Only elements tied with the exact key (bin still larger
  // than one after all four passes) need ordering by index, below. Histograms are double-buffered so that a pass
  // takes two barriers: the scan wave reads one buffer while the others clear the next.
  uint32_t prefix = 0, pmask = 0;
  uint32_t need = (uint32_t)j + 1u;
  uint32_t inbin = 0;
  hist[0][0][tid] = hist[0][1][tid] = hist[0][2][tid] = hist[0][3][tid] = 0u;
  __syncthreads();
  int buf = 0;
  for (int shift = 24; shift >= 0; shift -= 8) {
#pragma unroll
    for (int i = 0; i < NPT; ++i)
      if (tid + 256 * i < C && (ok[i] & pmask) == prefix)
        atomicAdd(&hist[buf][wave][(ok[i] >> shift) & 255u], 1u);
    __syncthreads();
    if (wave == 0) {
      // lane l owns digits 255-4l .. 252-4l (descending)
      uint32_t cnt[4], sum = 0;
#pragma unroll
      for (int q2 = 0; q2 < 4; ++q2) {
        const int dg = 255 - 4 * lane - q2;
        cnt[q2] = hist[buf][0][dg] + hist[buf][1][dg] + hist[buf][2][dg] + hist[buf][3][dg];
        sum += cnt[q2];
      }
      uint32_t incl = sum;  // inclusive prefix over lanes (higher digits first)
#pragma unroll
      for (int of = 1; of < 64; of <<= 1) {
        const uint32_t t = __shfl_up(incl, of, 64);
        if (lane >= of) incl += t;
      }
      uint32_t before = incl - sum;
#pragma unroll
      for (int q2 = 0; q2 < 4; ++q2) {
        if (before < need && before + cnt[q2] >= need) {
          sh_digit = 255u - 4u * lane - q2;
          sh_before = before;
          sh_n = cnt[q2];
        }
        before += cnt[q2];
      }
    } else {
      const int ow = wave - 1;  // waves 1-3 clear the other buffer (all four wave histograms)
      for (int i = ow * 64 + lane; i < 4 * 256; i += 3 * 64) (&hist[buf ^ 1][0][0])[i] = 0u;
    }
    __syncthreads();
    prefix |= sh_digit << shift;
    pmask |= 255u << shift;
    need -= sh_before;
    inbin = sh_n;
    buf ^= 1;
    if (inbin == 1u) break;
  }
  if (inbin == 1u) {
#pragma unroll
    for (int i = 0; i < NPT; ++i)
      if (tid + 256 * i < C && (ok[i] & pmask) == prefix) sh_c = tid + 256 * i;
    __syncthreads();
  } else {
  // the bin's members as (key, ~index) composites: descending composite order is the slot order
  __syncthreads();  // every wave has read the last bin count
  if (tid == 0) sh_n = 0u;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < NPT; ++i) {
    const int c = tid + 256 * i;
    if (c < C && (ok[i] & pmask) == prefix) {
      const uint32_t pos = atomicAdd(&sh_n, 1u);
      cand[pos] = ((uint64_t)ok[i] << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)c);
    }
  }
  __syncthreads();
  const uint32_t ncand = sh_n;
  if (ncand <= 64u) {
    if (wave == 0) {
      // lane e holds member e; its rank is the number of larger members, compared through scalar reads
      // (fully unrolled over the 64 lanes: empty lanes hold 0, which is never larger than a member)
      const uint64_t v = (uint32_t)lane < ncand ? cand[lane] : 0ull;
      const int vhi = (int)(v >> 32), vlo = (int)(uint32_t)v;
      uint32_t rank = 0;
#pragma unroll
      for (int f = 0; f < 64; ++f) {
        const uint64_t o = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane(vhi, f) << 32) |
                           (uint32_t)__builtin_amdgcn_readlane(vlo, f);
        rank += (o > v) ? 1u : 0u;
      }
      if ((uint32_t)lane < ncand && rank == need - 1u) sh_c = (int)(0xFFFFFFFFu - (uint32_t)(v & 0xFFFFFFFFull));
    }
  } else {
    // more than 64 elements share the exact key: their order is by index alone
    for (uint32_t e = tid; e < ncand; e += 256) {
      const uint64_t me = cand[e];
      uint32_t rank = 0;
      for (uint32_t f = 0; f < ncand; ++f) rank += (cand[f] > me) ? 1u : 0u;
      if (rank == need - 1u) sh_c = (int)(0xFFFFFFFFu - (uint32_t)(me & 0xFFFFFFFFull));
    }
  }
  __syncthreads();
  }
  const int c = sh_c;
  if (tid == 0 && sel) sel[(size_t)b * k + j] = c;

  // the cluster's candidate ids and their logits: group grp scores ids t = grp + 16 i, 8 ids per pass
  const int grp = tid >> 4, l16 = tid & 15;
  const int nper = vsc >> 4;  // ids per group (vsc % 16 == 0)
  const int32_t* ord = ordering + (size_t)c * vsc;
  const uint16_t* crow = Es + (size_t)c * vsc * H;
  uint64_t best = 0;
  for (int i0 = 0; i0 < nper; i0 += 8) {
    int idv[8];
    uint4 raw[8][HCH];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int t = min(grp + 16 * (i0 + u), vsc - 1);
      idv[u] = ord[t];
#pragma unroll
      for (int ch = 0; ch < HCH; ++ch)
        raw[u][ch] = *reinterpret_cast<const uint4*>(crow + (size_t)t * H + ch * 128 + l16 * 8);
    }
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    float acc[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc[u] = 0.f;
#pragma unroll
    for (int ch = 0; ch < HCH; ++ch) {
      const int col = ch * 128 + l16 * 8;
      float hf[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) hf[e] = hs[col + e];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        float ef[8];
        unpack8(raw[u][ch], ef);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[u] = fmaf(ef[e], hf[e], acc[u]);
      }
    }
    XR<8, 8>::run(acc, l16);  // over the 16 lanes of the group: lane l16 holds id (l16 >> 1) of the 8
    const int u = l16 >> 1;
    int idu = idv[0];
#pragma unroll
    for (int w2 = 1; w2 < 8; ++w2) idu = (u == w2) ? idv[w2] : idu;
    if ((l16 & 1) == 0 && i0 + u < nper) {
      const int t = grp + 16 * (i0 + u);
      const size_t slot = ((size_t)b * k + j) * vsc + t;
      if (ids) ids[slot] = idu;
      if (z) z[slot] = acc[0];
      if (logits) logits[(size_t)b * V + idu] = acc[0];
      best = u64_max(best, vid_key(acc[0], (uint32_t)idu));
    }
  }
  best = wave_max_u64(best);
  if (lane == 0) red[wave] = best;
  __syncthreads();
  if (tid == 0) keys[(size_t)b * k + j] = u64_max(u64_max(red[0], red[1]), u64_max(red[2], red[3]));
}

// ------------------------------------------------------------------------------------------------------------
// dense tied head: logits[b][v] = E[v] . h[b] for every token ([Guide] section 5: with use_ordered_embeddings off
// the head is the plain tied embedding; [MTP doc] "Variants supported": the large drafters use it), and the row's
// argmax folded into one (value, id) key per row by atomic max (keys must hold 0 beforehand).
//
// The table is streamed once per pass of up to 32 batch rows, as a GEMM on v_mfma_f32_16x16x32_bf16:
//   A = 16 table rows x 32 dims, loaded straight from HBM (lane l: row l%16, 8 dims at 8*(l/16) of each 32-dim
//       step, so each row's 64 contiguous bytes per step come from 4 lanes and two steps cover a 128-byte line);
//   B = the pass's hidden states from LDS, each fp32 value split into bf16 hi + lo (h = hi + lo within 2^-16
//       relative), two products per step, so the logits keep fp32-level accuracy;
//   D = 16 rows x 16 batch columns: lane l holds rows 4*(l/16) .. +3 of column l%16.
// A wave owns 32-row groups (two 16-row tiles) over the whole hidden dimension: no cross-wave reduction. Its loads
// run in chunks of P steps, double-buffered, and the next group's first chunk is requested during the current
// group's last chunk (from a clamped group index, so the issue count never depends on data).
// grid (blocks, ceil(B / 32)), 1024 threads; NC = batch columns per pass (16 or 32), H = 256 * NPL.

template <int NC, int NPL>
__global__ __launch_bounds__(1024) void k_head_dense(int B, int V, const uint16_t* E, const float* h,
                                                     float* __restrict__ logits, uint64_t* __restrict__ keys) {
  constexpr int H = NPL * 256, KSTEPS = H / 32, LROW = H + 8, NBT = NC / 16;
  // tiles per group, steps per chunk (fewer with 32 columns, whose operands take more registers), chunks per group
  constexpr int RT = 2, P = NC == 32 ? 2 : 4, NCH = KSTEPS / P;
  static_assert(NCH % 2 == 0, "chunks alternate between the two buffers");
  constexpr int NW = 16;
  __shared__ __attribute__((aligned(16))) uint16_t hs[2][NC][LROW];  // [hi / lo][column][dim], rows padded by 16 B
  __shared__ uint64_t red[NW][NC];
  const int wave = wave_id(), lane = lane_id(), tid = threadIdx.x;
  const int n = lane & 15, g4 = lane >> 4;
  const int c0 = blockIdx.y * NC;
  const int ngroups = (V + 31) / 32;
  const int gstride = gridDim.x * NW;
  int grp = blockIdx.x * NW + wave;

  // lane's pieces of row 32 gq + 16 r + n (clamped to V - 1) start at element 8 g4 of the row; step s adds 32 s.
  // Offsets, not pointers, are carried between groups: pointers carried through the loop lose their global
  // address space and become flat loads.
  auto rows_of = [&](int gq, size_t (&ro)[RT]) {
#pragma unroll
    for (int r = 0; r < RT; ++r) ro[r] = (size_t)min(gq * 32 + r * 16 + n, V - 1) * H + 8 * g4;
  };
  auto load = [&](uint4 (&a)[P][RT], const size_t (&ro)[RT], int c) {
#pragma unroll
    for (int p = 0; p < P; ++p)
#pragma unroll
      for (int r = 0; r < RT; ++r) a[p][r] = ld_global16(E + ro[r] + (c * P + p) * 32);
  };
  uint4 a0[P][RT], a1[P][RT];
  size_t rp[RT];
  rows_of(min(grp, ngroups - 1), rp);
  load(a0, rp, 0);

  // stage the pass's hidden states as bf16 hi + lo (columns past B are zero)
  constexpr int NV4 = NC * H / 4 / 1024;  // float4 per thread
  static_assert(NV4 >= 1 && NC * H % 4096 == 0, "staging covers the columns exactly");
  float4 hv[NV4];
#pragma unroll
  for (int i = 0; i < NV4; ++i) {
    const int e = (tid + i * 1024) * 4, col = e / H, k = e % H;
    const int b = min(c0 + col, B - 1);
    hv[i] = *reinterpret_cast<const float4*>(h + (size_t)b * H + k);
  }
#pragma unroll
  for (int i = 0; i < NV4; ++i) {
    const int e = (tid + i * 1024) * 4, col = e / H, k = e % H;
    const bool live = c0 + col < B;
    const float f[4] = {hv[i].x, hv[i].y, hv[i].z, hv[i].w};
    uint16_t hi[4], lo[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float v = live ? f[j] : 0.f;
      hi[j] = f2bf(v);
      lo[j] = f2bf(v - bf2f(hi[j]));
    }
    *reinterpret_cast<uint2*>(&hs[0][col][k]) =
        make_uint2(hi[0] | ((uint32_t)hi[1] << 16), hi[2] | ((uint32_t)hi[3] << 16));
    *reinterpret_cast<uint2*>(&hs[1][col][k]) =
        make_uint2(lo[0] | ((uint32_t)lo[1] << 16), lo[2] | ((uint32_t)lo[3] << 16));
  }
  __syncthreads();

  float best[NBT];
  int bid[NBT];
#pragma unroll
  for (int t = 0; t < NBT; ++t) {
    best[t] = -INFINITY;
    bid[t] = -1;
  }

  auto compute = [&](const uint4 (&a)[P][RT], int c, f32x4 (&acc)[RT][NBT]) {
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int k = (c * P + p) * 32 + 8 * g4;
      uint4 bh[NBT], bl[NBT];
#pragma unroll
      for (int t = 0; t < NBT; ++t) {
        bh[t] = *reinterpret_cast<const uint4*>(&hs[0][t * 16 + n][k]);
        bl[t] = *reinterpret_cast<const uint4*>(&hs[1][t * 16 + n][k]);
      }
#pragma unroll
      for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int t = 0; t < NBT; ++t)
          acc[r][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[p][r]),
                                                              __builtin_bit_cast(bf16x8, bh[t]), acc[r][t], 0, 0, 0);
#pragma unroll
      for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int t = 0; t < NBT; ++t)
          acc[r][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[p][r]),
                                                              __builtin_bit_cast(bf16x8, bl[t]), acc[r][t], 0, 0, 0);
    }
  };

  while (grp < ngroups) {  // wave-uniform
    size_t rn[RT];
    rows_of(min(grp + gstride, ngroups - 1), rn);
    f32x4 acc[RT][NBT];
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int t = 0; t < NBT; ++t) acc[r][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NCH; c += 2) {
      // the order as written (each buffer refilled right after its last use) is what bounds the live registers:
      // the scheduler must not hoist later loads above the products
      load(a1, rp, c + 1);
      __builtin_amdgcn_sched_barrier(0);
      compute(a0, c, acc);
      __builtin_amdgcn_sched_barrier(0);
      if (c + 2 < NCH)
        load(a0, rp, c + 2);
      else
        load(a0, rn, 0);
      __builtin_amdgcn_sched_barrier(0);
      compute(a1, c + 1, acc);
      __builtin_amdgcn_sched_barrier(0);
    }
    // epilogue: full logits and the running (value, id) best per column; rows visited in increasing order, so a
    // strict comparison keeps the lowest id among equal values
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      const int row0 = grp * 32 + r * 16 + 4 * g4;
      if (grp * 32 + r * 16 < V) {  // V % 16 == 0: a tile is wholly inside or outside the table
#pragma unroll
        for (int t = 0; t < NBT; ++t) {
          const int col = c0 + t * 16 + n;
          const f32x4 v = acc[r][t];
          if (logits && col < B)
            *reinterpret_cast<float4*>(logits + (size_t)col * V + row0) = make_float4(v[0], v[1], v[2], v[3]);
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (v[i] > best[t]) {
              best[t] = v[i];
              bid[t] = row0 + i;
            }
        }
      }
    }
    grp += gstride;
#pragma unroll
    for (int r = 0; r < RT; ++r) rp[r] = rn[r];
  }

  // block-wide best per column, then one atomic max per (block, column)
#pragma unroll
  for (int t = 0; t < NBT; ++t) {
    uint64_t kk = bid[t] >= 0 ? vid_key(best[t], (uint32_t)bid[t]) : 0ull;
#pragma unroll
    for (int o = 16; o < 64; o <<= 1) {
      const uint32_t lo = __shfl_xor((uint32_t)kk, o, 64);
      const uint32_t hi = __shfl_xor((uint32_t)(kk >> 32), o, 64);
      kk = u64_max(kk, ((uint64_t)hi << 32) | lo);
    }
    if (g4 == 0) red[wave][t * 16 + n] = kk;
  }
  __syncthreads();
  if (tid < NC && c0 + tid < B) {
    uint64_t m = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) m = u64_max(m, red[w][tid]);
    if (m) atomicMax(reinterpret_cast<unsigned long long*>(keys + c0 + tid), (unsigned long long)m);
  }
}

__global__ void k_zero_u64(uint64_t* __restrict__ p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0ull;
}

// Head table in cluster order: out[r] = E[ordering[r]], rows of H bf16 (H % 8 == 0); grid ceil(V / 8), 256 threads,
// 32 threads per row.
__global__ __launch_bounds__(256) void k_gather_rows(const uint16_t* __restrict__ E, const int32_t* __restrict__ ordering,
                                                     uint16_t* __restrict__ out, int V, int H) {
  const int r = blockIdx.x * 8 + (threadIdx.x >> 5);
  if (r >= V) return;
  const uint4* src = reinterpret_cast<const uint4*>(E + (size_t)ordering[r] * H);
  uint4* dst = reinterpret_cast<uint4*>(out + (size_t)r * H);
  for (int i = threadIdx.x & 31; i < H / 8; i += 32) dst[i] = src[i];
}

// grid B, 64 threads
__global__ void k_final(int k, const uint64_t* __restrict__ keys, int32_t* __restrict__ next,
                        int32_t* __restrict__ out2, int stride2) {
  const int b = blockIdx.x, lane = threadIdx.x;
  const uint64_t kv = (lane < k) ? keys[(size_t)b * k + min(lane, k - 1)] : 0ull;
  const int32_t id = key_id(wave_max_u64(kv));
  if (lane == 0) {
    next[b] = id;
    if (out2) out2[(size_t)b * stride2] = id;
  }
}

__global__ void k_fill(float4* __restrict__ p, size_t n4, float* __restrict__ tail, int ntail) {
  const float4 v = make_float4(-1e30f, -1e30f, -1e30f, -1e30f);
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) p[i] = v;
  if (blockIdx.x == 0 && (int)threadIdx.x < ntail) tail[threadIdx.x] = -1e30f;
}

int row_groups(int B) { return (B + kRG - 1) / kRG; }

// MTPD_ATTN_VALU=1 selects the vector-ALU attention for every shape (kept for comparison and as the general path).
// Read at each launch (a captured graph keeps the kernel it was captured with).
bool getenv_no_mfma() {
  const char* e = getenv("MTPD_ATTN_VALU");
  return e && e[0] == '1';
}

// Timing events for the next launch only (see set_next_launch_events).
thread_local hipEvent_t t_ev_start = nullptr, t_ev_stop = nullptr;

// Launch `k` on `s`; when timing events are pending they are attached to this launch (recorded by the runtime at
// the kernel's start and end) and consumed.
template <typename... P, typename... A>
hipError_t go(void (*k)(P...), dim3 grid, dim3 block, size_t shmem, hipStream_t s, A... a) {
  static_assert(sizeof...(P) == sizeof...(A), "argument count");
  if (t_ev_start || t_ev_stop) {
    hipEvent_t e0 = t_ev_start, e1 = t_ev_stop;
    t_ev_start = t_ev_stop = nullptr;
    hipExtLaunchKernelGGL(k, grid, block, (uint32_t)shmem, s, e0, e1, 0u, static_cast<P>(a)...);
  } else {
    k<<<grid, block, shmem, s>>>(static_cast<P>(a)...);
  }
  return hipGetLastError();
}

}  // namespace

// ------------------------------------------------------------------------------------------------------------
// launchers

void set_next_launch_events(hipEvent_t start, hipEvent_t stop) {
  t_ev_start = start;
  t_ev_stop = stop;
}

hipError_t launch_pre(hipStream_t s, int B, int Bb, int H, int V, const uint16_t* th, TokenSource ts,
                      const uint16_t* emb, float escale, const uint16_t* w_pre, float* x) {
  const dim3 grid((H + 3) / 4, row_groups(B));
  const int nch = Bb / 128;  // 256-wide chunks of K = 2 Bb
#define MTPD_PRE(NWV_, CPW_) \
  return go(k_pre<NWV_, CPW_>, grid, NWV_ * 64, 0, s, B, Bb, H, V, th, ts, emb, escale, w_pre, x)
  if (nch <= 32) {
    switch ((nch + 3) / 4) {
      case 1: MTPD_PRE(4, 1);
      case 2: MTPD_PRE(4, 2);
      case 3: MTPD_PRE(4, 3);
      case 4: MTPD_PRE(4, 4);
      case 5: MTPD_PRE(4, 5);
      case 6: MTPD_PRE(4, 6);
      case 7: MTPD_PRE(4, 7);
      case 8: MTPD_PRE(4, 8);
    }
  } else {
    switch ((nch + 7) / 8) {
      case 5: MTPD_PRE(8, 5);
      case 6: MTPD_PRE(8, 6);
      case 7: MTPD_PRE(8, 7);
      case 8: MTPD_PRE(8, 8);
    }
  }
#undef MTPD_PRE
  return hipErrorInvalidValue;
}

// H = 64 NPL for the kernels with a norm prologue (hidden in {256, 512, 768, 1024})
#define MTPD_BY_NPL(H_, CALL)        \
  switch ((H_) / 64) {               \
    case 4: { constexpr int NPL = 4; CALL; }   \
    case 8: { constexpr int NPL = 8; CALL; }   \
    case 12: { constexpr int NPL = 12; CALL; } \
    case 16: { constexpr int NPL = 16; CALL; } \
  }                                  \
  return hipErrorInvalidValue;

hipError_t launch_qproj(hipStream_t s, int B, int H, int QD, Residual res, const uint16_t* w_norm, float eps,
                        const uint16_t* w_q, float* q) {
  const dim3 grid((QD + 15) / 16, row_groups(B));
  MTPD_BY_NPL(H, return go(k_qproj<NPL>, grid, 256, 0, s, B, QD, res, w_norm, eps, w_q, q))
}

hipError_t launch_dense(hipStream_t s, int B, int K, int N, const float* X, const uint16_t* w, float* y) {
  const dim3 grid((N + 3) / 4, row_groups(B));
  switch (K / 256) {
#define MTPD_DENSE(IT_) \
  case IT_:             \
    return go(k_dense<IT_>, grid, 256, 0, s, B, N, X, w, y);
    MTPD_DENSE(1) MTPD_DENSE(2) MTPD_DENSE(3) MTPD_DENSE(4) MTPD_DENSE(5) MTPD_DENSE(6) MTPD_DENSE(7) MTPD_DENSE(8)
    MTPD_DENSE(9) MTPD_DENSE(10) MTPD_DENSE(11) MTPD_DENSE(12) MTPD_DENSE(13) MTPD_DENSE(14) MTPD_DENSE(15)
    MTPD_DENSE(16)
#undef MTPD_DENSE
  }
  return hipErrorInvalidValue;
}

hipError_t launch_scores(hipStream_t s, int B, int H, int C, const float* h, const uint16_t* w_cen, float* scores) {
  return launch_dense(s, B, H, C, h, w_cen, scores);
}

hipError_t launch_ffn(hipStream_t s, int B, int H, int F, Residual res, const uint16_t* w_norm, float eps,
                      const uint16_t* w_gate, const uint16_t* w_up, float* m, FillRange fill) {
  const dim3 grid((F + 15) / 16, row_groups(B));
  const int nd = res.delta ? res.nd : 1;
#define MTPD_FFN(ND_) \
  MTPD_BY_NPL(H, return go(k_ffn<NPL, ND_>, grid, 256, 0, s, B, F, res, w_norm, eps, w_gate, w_up, m, fill))
  if (nd <= 1) {
    MTPD_FFN(1)
  } else if (nd <= 2) {
    MTPD_FFN(2)
  } else if (nd <= 4) {
    MTPD_FFN(4)
  } else if (nd <= 8) {
    MTPD_FFN(8)
  } else {
    MTPD_FFN(16)
  }
#undef MTPD_FFN
}

hipError_t launch_post(hipStream_t s, int B, int H, int Bb, int C, Residual res, const uint16_t* w_out, float eps,
                       const uint16_t* w_post, const uint16_t* w_cen, float* h_out, uint16_t* hidden_out,
                       float* scores, uint64_t* keys_zero) {
  const dim3 grid((Bb + C + 31) / 32, row_groups(B));
  MTPD_BY_NPL(H, return go(k_post<NPL>, grid, 256, 0, s, B, Bb, C, res, w_out, eps, w_post, w_cen, h_out,
                           hidden_out, scores, keys_zero))
}
#undef MTPD_BY_NPL

hipError_t launch_attn(hipStream_t s, int B, int nh, int nkv, int hd, const float* q, const uint16_t* qnorm,
                       float eps, const float* rope, int type, const uint16_t* K, const uint16_t* V, int cap,
                       const RowWindows& win, int nsplit, float scale, float* pacc, float* pml, float* o) {
  dim3 grid(nsplit, B * nkv);
  const float sl2 = scale * 1.4426950408889634f;
  const int G = nh / nkv;
  if (hd == 256 && G <= 8 && !getenv_no_mfma()) {
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

hipError_t launch_oproj(hipStream_t s, int B, int N, int QD, int hd, int nh, int nsplit, const float* o,
                        const float* pacc, const float* pml, const uint16_t* W, float* t) {
  const dim3 grid((N + 63) / 64, QD / 256, B);
#define MTPD_OPROJ(NS_) return go(k_oproj<NS_>, grid, 256, 0, s, N, QD, hd, nh, nsplit, o, pacc, pml, W, t)
  if (nsplit <= 1) MTPD_OPROJ(1);
  if (nsplit <= 2) MTPD_OPROJ(2);
  if (nsplit <= 4) MTPD_OPROJ(4);
  if (nsplit <= 8) MTPD_OPROJ(8);
  if (nsplit <= 16) MTPD_OPROJ(16);
  MTPD_OPROJ(32);
#undef MTPD_OPROJ
}

hipError_t launch_head(hipStream_t s, int B, int C, int k, int vsc, int H, const float* scores,
                       const int32_t* ordering, const uint16_t* Es, const float* h, int32_t* sel, int32_t* ids,
                       float* z, float* logits, size_t V, uint64_t* keys) {
  const dim3 grid(k, B);
  const int npt = C <= 256 ? 1 : C <= 512 ? 2 : C <= 1024 ? 4 : C <= 2048 ? 8 : 16;
#define MTPD_HEAD(NPT_, HCH_)                                                                                 \
  if (npt == NPT_ && H == HCH_ * 128)                                                                         \
    return go(k_head<NPT_, HCH_>, grid, 256, 0, s, C, k, vsc, scores, ordering, Es, h, sel, ids, z, logits, V, \
              keys);
  MTPD_HEAD(1, 2) MTPD_HEAD(2, 2) MTPD_HEAD(4, 2) MTPD_HEAD(8, 2) MTPD_HEAD(16, 2)
  MTPD_HEAD(1, 4) MTPD_HEAD(2, 4) MTPD_HEAD(4, 4) MTPD_HEAD(8, 4) MTPD_HEAD(16, 4)
  MTPD_HEAD(1, 6) MTPD_HEAD(2, 6) MTPD_HEAD(4, 6) MTPD_HEAD(8, 6) MTPD_HEAD(16, 6)
  MTPD_HEAD(1, 8) MTPD_HEAD(2, 8) MTPD_HEAD(4, 8) MTPD_HEAD(8, 8) MTPD_HEAD(16, 8)
#undef MTPD_HEAD
  return hipErrorInvalidValue;
}

hipError_t launch_head_dense(hipStream_t s, int B, int V, int H, const uint16_t* E, const float* h, float* logits,
                             uint64_t* keys) {
  const int ngroups = (V + 31) / 32;
  const int nc = B <= 16 ? 16 : 32;
  const int nblk = (ngroups + 15) / 16;
  const dim3 grid(nblk < 256 ? nblk : 256, (B + nc - 1) / nc);
#define MTPD_HD(NC_, NPL_) \
  if (nc == NC_ && H == NPL_ * 256) return go(k_head_dense<NC_, NPL_>, grid, 1024, 0, s, B, V, E, h, logits, keys);
  MTPD_HD(16, 1) MTPD_HD(16, 2) MTPD_HD(16, 3) MTPD_HD(16, 4)
  MTPD_HD(32, 1) MTPD_HD(32, 2) MTPD_HD(32, 3) MTPD_HD(32, 4)
#undef MTPD_HD
  return hipErrorInvalidValue;
}

hipError_t launch_zero_keys(hipStream_t s, uint64_t* keys, int n) {
  return go(k_zero_u64, (n + 255) / 256, 256, 0, s, keys, n);
}

hipError_t launch_gather_rows(hipStream_t s, const uint16_t* E, const int32_t* ordering, uint16_t* out, int V,
                              int H) {
  return go(k_gather_rows, (V + 7) / 8, 256, 0, s, E, ordering, out, V, H);
}

hipError_t launch_final(hipStream_t s, int B, int k, const uint64_t* keys, int32_t* next, int32_t* out2,
                        int stride2) {
  return go(k_final, B, 64, 0, s, k, keys, next, out2, stride2);
}

hipError_t launch_fill(hipStream_t s, float* logits, size_t n) {
  const size_t n4 = n / 4;
  const int ntail = (int)(n - n4 * 4);
  size_t grid = (n4 + 255) / 256;
  if (grid > 4096) grid = 4096;
  if (grid < 1) grid = 1;
  return go(k_fill, (unsigned)grid, 256, 0, s, reinterpret_cast<float4*>(logits), n4, logits + n4 * 4, ntail);
}

}  // namespace mtpd
