// Dense stages for large batches (32 rows and more): the drafter's projections there are dense contractions
// (M = batch), so they run as streaming matrix-core GEMMs that read each weight matrix once per 16 batch rows,
// after one residual + norm kernel per stage (instead of every block repeating the stage's prologue).
//
// Pages cited (by title; sections as headed on each page):
//   [MTP doc]    "Gemma 4 Multi-Token Prediction (MTP) drafter" (llama.cpp fork, gemma4-assistant.md)
//   [Inventory]  "Gemma 4 Assistant (MTP drafter) - tensor inventory (Stage 0)"
//   [Guide]      "Gemma 4 Assistant 使用指南：用 MTP 投机解码与 KV Sharing 加速 Gemma 4 推理" (gitcode blog)
//
// The arithmetic is the same as the small-batch kernels' ([MTP doc] "What it is", "Tensor schema": pre_projection,
// q / o projections, GeGLU FFN, sandwich norms, layer scalar, post_projection; [Inventory] "Centroid / ordered
// embeddings LM head" step 1: centroid scores): bf16 weights, fp32 activations and accumulation. On the matrix cores
// each fp32 activation enters as bf16 hi + lo (h = hi + lo within 2^-16 relative), two products per step.
#include "device.h"

namespace mtpd {
namespace {

// ------------------------------------------------------------------------------------------------------------
// Y = W X^T over a K chunk: grid (ceil(N / (64 / WPT)), K / KC, ceil(B / 16)), 256 threads. Block: 64 / WPT output
// rows x 16 batch rows x the K chunk blockIdx.y. The chunk of X (16 rows) is staged in LDS as bf16 hi + lo. WPT
// waves share each 16-row tile, each streaming its tile's weight rows over its own KC / WPT of the chunk (A operand
// of v_mfma_f32_16x16x32_bf16: lane l reads row l%16, 8 dims at 8 (l/16) of each 32-dim step) in double-buffered
// chunks of P steps, so that a wave's loads take few round trips; the WPT partial sums meet in LDS in a fixed order.
// Sources of X: SRC_F32 fp32 rows [B][K]; SRC_PRE the pre_projection input [target hidden ; escale * embedding of
// the row's token] from bf16 tables (tokens already resolved). Epilogues: EPI_F32 partial [kc][B][N] fp32;
// EPI_BF16 bf16 [B][N] (K in one chunk); EPI_GEGLU gelu_tanh(W x) * (W2 x) fp32 [B][N] (K in one chunk).

enum { SRC_F32 = 0, SRC_PRE = 1 };
enum { EPI_F32 = 0, EPI_BF16 = 1, EPI_GEGLU = 2 };

struct GemmSrc {
  const float* x;          // SRC_F32: [B][K]
  const uint16_t* th;      // SRC_PRE: target hidden [B][Bb]
  const uint16_t* emb;     // SRC_PRE: embedding table [V][Bb]
  TokenSource ts;          // SRC_PRE: the rows' tokens (the caller's, or the previous step's argmax from its keys)
  int V;                   // SRC_PRE: vocabulary (tokens are clamped into [0, V))
  int Bb;                  // SRC_PRE: backbone width (K = 2 Bb)
  float escale;            // SRC_PRE: factor on the embedding half
};

template <int KC, int WPT, int SRC, int EPI>
__global__ __launch_bounds__(256) void k_gemm(int B, int N, int K, GemmSrc src, const uint16_t* W, const uint16_t* W2,
                                              float* Y, uint16_t* Yb, FillRange fill) {
  constexpr int NC = 16, KSTEPS = KC / 32, LROW = KC + 8;
  constexpr int WSTEPS = KSTEPS / WPT;  // steps per wave (WPT waves per 16-row tile)
  constexpr int NW2 = EPI == EPI_GEGLU ? 2 : 1;
  // steps per load chunk: 8 (4 with the two GeGLU matrices), fewer when the wave's steps do not divide
  constexpr int PMAX = EPI == EPI_GEGLU ? 4 : 8;
  constexpr int P = WSTEPS % PMAX == 0 ? PMAX : (WSTEPS % 4 == 0 ? 4 : (WSTEPS % 2 == 0 ? 2 : 1));
  static_assert(KC % 256 == 0 && WSTEPS % P == 0, "whole load chunks");
  __shared__ __attribute__((aligned(16))) uint16_t xs[2][NC][LROW];  // [hi / lo][batch row][dim]
  __shared__ __attribute__((aligned(16))) f32x4 part[4][NW2][64];     // partial sums of the waves of a tile
  const int wave = wave_id(), lane = lane_id(), tid = threadIdx.x;
  const int hq = lane & 15, kq = lane >> 4;
  const int n0 = blockIdx.x * (64 / WPT) + (wave / WPT) * 16;
  const int kw = (wave % WPT) * (KC / WPT);  // the wave's part of the chunk
  const int kc = blockIdx.y, kbase = kc * KC;
  const int c0 = blockIdx.z * NC;
  const uint16_t* wrow[2];
  wrow[0] = W + (size_t)min(n0 + hq, N - 1) * K + kbase + kw + 8 * kq;
  wrow[1] = (EPI == EPI_GEGLU ? W2 : W) + (size_t)min(n0 + hq, N - 1) * K + kbase + kw + 8 * kq;

  uint4 a[2][NW2][P];  // [buffer][matrix][step]
  auto load = [&](int bf, int ch) {
#pragma unroll
    for (int m = 0; m < NW2; ++m)
#pragma unroll
      for (int p = 0; p < P; ++p) a[bf][m][p] = ld_global16(wrow[m] + (ch * P + p) * 32);
  };
  load(0, 0);

  // the block's share of the logits fill ([Inventory] "Centroid / ordered embeddings LM head", step 5: the -1e30 base
  // row), written while the weight loads are in flight (streaming stores: nothing reads the row before the head)
  if (fill.logits) {
    const size_t nblk = (size_t)gridDim.x * gridDim.y * gridDim.z;
    const size_t bid = ((size_t)blockIdx.z * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x;
    const size_t total = fill.end - fill.begin;
    const size_t per = ((total + nblk - 1) / nblk + 3) & ~(size_t)3;
    const size_t a = fill.begin + bid * per;
    const size_t e = a + per < fill.end ? a + per : fill.end;
    if (a < e) {
      const f32x4 v = f32x4{-1e30f, -1e30f, -1e30f, -1e30f};
      size_t i = a + tid * 4;
      for (; i + 4 <= e; i += 1024) __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(fill.logits + i));
      for (; i < e; ++i) __builtin_nontemporal_store(-1e30f, fill.logits + i);
    }
  }

  // stage the X chunk: 16 rows x KC, rows past B are zero
  constexpr int NV4 = NC * KC / 4 / 256;  // float4 (or 4 bf16) per thread
  float xf[NV4][4];
  if constexpr (SRC == SRC_F32) {
#pragma unroll
    for (int i = 0; i < NV4; ++i) {
      const int e = (tid + i * 256) * 4, r = e / KC, k = e % KC;
      const float4 v = *reinterpret_cast<const float4*>(src.x + (size_t)min(c0 + r, B - 1) * K + kbase + k);
      xf[i][0] = v.x; xf[i][1] = v.y; xf[i][2] = v.z; xf[i][3] = v.w;
    }
  } else {
    // the tile's 16 tokens, one row per wave at a time: the caller's, or the argmax of the row's keys from the
    // previous step (recorded by the blocks of the first output tile and chunk), clamped into [0, V)
    __shared__ int tks[NC];
    {
      const TokenSource& ts = src.ts;
#pragma unroll
      for (int q = 0; q < NC / 4; ++q) {
        const int r = (tid >> 6) * (NC / 4) + q, b = min(c0 + r, B - 1);
        const uint64_t kraw = ts.keys[(size_t)b * ts.k + min(lane, ts.k - 1)];
        int t = ts.tok[b];
        if (ts.use_keys) {
          t = key_id(wave_max_u64(lane < ts.k ? kraw : 0ull));
          if (lane == 0 && blockIdx.x == 0 && blockIdx.y == 0 && c0 + r < B) {
            if (ts.out) ts.out[(size_t)b * ts.out_stride] = t;
            if (ts.next) ts.next[b] = t;
          }
        }
        if (lane == 0) tks[r] = t < 0 ? 0 : (t >= src.V ? src.V - 1 : t);
      }
      __syncthreads();
    }
    // then every row load unconditionally (a select picks the table), so that the loads issue together instead of
    // one branch, load and wait per element
    int tk[NV4];
#pragma unroll
    for (int i = 0; i < NV4; ++i) tk[i] = tks[((tid + i * 256) * 4) / KC];
    uint2 w[NV4];
#pragma unroll
    for (int i = 0; i < NV4; ++i) {
      const int e = (tid + i * 256) * 4, r = e / KC, k = e % KC;
      const int kk = kbase + k;  // Bb % 256 == 0: 4 dims lie in one half
      const bool hid = kk < src.Bb;
      const size_t oh = (size_t)min(c0 + r, B - 1) * src.Bb + kk;
      const size_t oe = (size_t)tk[i] * src.Bb + (kk - src.Bb);
      const uint16_t* ptr = hid ? src.th + oh : src.emb + oe;
      w[i] = *reinterpret_cast<const uint2*>(ptr);
    }
#pragma unroll
    for (int i = 0; i < NV4; ++i) {
      const int kk = kbase + ((tid + i * 256) * 4) % KC;
      const float sc = kk < src.Bb ? 1.0f : src.escale;
      unpack4(w[i], xf[i]);
#pragma unroll
      for (int j = 0; j < 4; ++j) xf[i][j] *= sc;
    }
  }
#pragma unroll
  for (int i = 0; i < NV4; ++i) {
    const int e = (tid + i * 256) * 4, r = e / KC, k = e % KC;
    const bool live = c0 + r < B;
    uint32_t hi[2], lo[2];
    split_bf16x2(live ? xf[i][0] : 0.f, live ? xf[i][1] : 0.f, hi[0], lo[0]);
    split_bf16x2(live ? xf[i][2] : 0.f, live ? xf[i][3] : 0.f, hi[1], lo[1]);
    *reinterpret_cast<uint2*>(&xs[0][r][k]) = make_uint2(hi[0], hi[1]);
    *reinterpret_cast<uint2*>(&xs[1][r][k]) = make_uint2(lo[0], lo[1]);
  }
  __syncthreads();

  f32x4 acc[NW2];
#pragma unroll
  for (int m = 0; m < NW2; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](int bf, int ch) {
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int k = kw + (ch * P + p) * 32 + 8 * kq;
      const uint4 bh = *reinterpret_cast<const uint4*>(&xs[0][hq][k]);
      const uint4 bl = *reinterpret_cast<const uint4*>(&xs[1][hq][k]);
#pragma unroll
      for (int m = 0; m < NW2; ++m) {
        acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[bf][m][p]),
                                                         __builtin_bit_cast(bf16x8, bh), acc[m], 0, 0, 0);
        acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[bf][m][p]),
                                                         __builtin_bit_cast(bf16x8, bl), acc[m], 0, 0, 0);
      }
    }
  };
  constexpr int NCH = WSTEPS / P;
#pragma unroll
  for (int ch = 0; ch < NCH; ch += 2) {
    if (ch + 1 < NCH) load(1, ch + 1);
    __builtin_amdgcn_sched_barrier(0);
    compute(0, ch);
    __builtin_amdgcn_sched_barrier(0);
    if (ch + 2 < NCH) load(0, ch + 2);
    __builtin_amdgcn_sched_barrier(0);
    if (ch + 1 < NCH) compute(1, ch + 1);
    __builtin_amdgcn_sched_barrier(0);
  }

  // the tile's WPT partial sums, added in wave order by the tile's first wave
  if constexpr (WPT > 1) {
#pragma unroll
    for (int m = 0; m < NW2; ++m) part[wave][m][lane] = acc[m];
    __syncthreads();
    if (wave % WPT != 0) return;
#pragma unroll
    for (int m = 0; m < NW2; ++m) {
      f32x4 sum = part[wave][m][lane];
#pragma unroll
      for (int w = 1; w < WPT; ++w) {
        const f32x4 v = part[wave + w][m][lane];
        sum = f32x4{sum[0] + v[0], sum[1] + v[1], sum[2] + v[2], sum[3] + v[3]};
      }
      acc[m] = sum;
    }
  }
  // D: rows n0 + 4 kq + i, batch column c0 + hq
  const int c = c0 + hq, n = n0 + 4 * kq;
  if (c < B && n0 < N) {  // N % 16 == 0: a wave's 16 rows are wholly inside or outside
    if constexpr (EPI == EPI_F32) {
      *reinterpret_cast<float4*>(Y + ((size_t)kc * B + c) * N + n) = make_float4(acc[0][0], acc[0][1], acc[0][2], acc[0][3]);
    } else if constexpr (EPI == EPI_BF16) {
      *reinterpret_cast<uint2*>(Yb + (size_t)c * N + n) =
          make_uint2(f2bf2(acc[0][0], acc[0][1]), f2bf2(acc[0][2], acc[0][3]));
    } else {
      float mv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) mv[i] = gelu_tanh(acc[0][i]) * acc[NW2 - 1][i];
      *reinterpret_cast<float4*>(Y + (size_t)c * N + n) = make_float4(mv[0], mv[1], mv[2], mv[3]);
    }
  }
}

// ------------------------------------------------------------------------------------------------------------
// Residual + norms of one row per block (256 threads, H = 256 HPT): x = sum of the nx partials of xp (stride xs);
// with a delta, x = (x + RMSNorm(sum of the nd partials of the delta; w_delta)) * scale; x_new = x (when set);
// u = RMSNorm(x; w_norm). Partial counts are template maxima NX / ND (loads clamped, surplus weighted by zero).

template <int HPT>
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  if (lane_id() == 0) red[wave_id()] = v;
  __syncthreads();
  const float s = (red[0] + red[1]) + (red[2] + red[3]);
  __syncthreads();
  return s;
}

template <int HPT, int NX, int ND>
__global__ __launch_bounds__(256) void k_rownorm(int B, const float* xp, int nx, size_t xs, const float* delta,
                                                 int nd, size_t ds, const uint16_t* w_delta, float scale,
                                                 const uint16_t* w_norm, float eps, float* x_new, float* u,
                                                 uint64_t* keys_zero) {
  constexpr int H = HPT * 256;
  __shared__ float red[4];
  const int b = blockIdx.x, tid = threadIdx.x;
  // every load first and unconditionally, so that none waits behind a branch: without a delta the delta slots read
  // the x partials (valid memory; the values are not used) and the delta weights read w_norm
  const bool hasd = delta != nullptr;
  const float* dsrc = hasd ? delta : xp;
  const size_t dstr = hasd ? ds : xs;
  const int ndl = hasd ? nd : nx;
  const uint16_t* wdsrc = hasd ? w_delta : w_norm;
  float xv[NX][HPT], dv[ND][HPT], wd[HPT], wn[HPT];
#pragma unroll
  for (int p = 0; p < NX; ++p)
#pragma unroll
    for (int i = 0; i < HPT; ++i) xv[p][i] = xp[(size_t)min(p, nx - 1) * xs + (size_t)b * H + tid + 256 * i];
#pragma unroll
  for (int p = 0; p < ND; ++p)
#pragma unroll
    for (int i = 0; i < HPT; ++i) dv[p][i] = dsrc[(size_t)min(p, ndl - 1) * dstr + (size_t)b * H + tid + 256 * i];
#pragma unroll
  for (int i = 0; i < HPT; ++i) {
    wd[i] = bf2f(wdsrc[tid + 256 * i]);
    wn[i] = bf2f(w_norm[tid + 256 * i]);
  }
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  float x[HPT];
#pragma unroll
  for (int i = 0; i < HPT; ++i) {
    float s = 0.f;
#pragma unroll
    for (int p = 0; p < NX; ++p) s += p < nx ? xv[p][i] : 0.f;
    x[i] = s;
  }
  if (hasd) {
    float d[HPT], ss = 0.f;
#pragma unroll
    for (int i = 0; i < HPT; ++i) {
      float s = 0.f;
#pragma unroll
      for (int p = 0; p < ND; ++p) s += p < nd ? dv[p][i] : 0.f;
      d[i] = s;
      ss = fmaf(s, s, ss);
    }
    const float r = rsqrt_hw(block_sum<HPT>(ss, red) / (float)H + eps);
#pragma unroll
    for (int i = 0; i < HPT; ++i) x[i] = (x[i] + d[i] * r * wd[i]) * scale;
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < HPT; ++i) {
    if (x_new) x_new[(size_t)b * H + tid + 256 * i] = x[i];
    ss = fmaf(x[i], x[i], ss);
  }
  const float r = rsqrt_hw(block_sum<HPT>(ss, red) / (float)H + eps);
#pragma unroll
  for (int i = 0; i < HPT; ++i) u[(size_t)b * H + tid + 256 * i] = x[i] * r * wn[i];
  if (keys_zero && tid == 0) keys_zero[b] = 0ull;
}

// ------------------------------------------------------------------------------------------------------------
// Merge of the key-range split partials of the attention: o[b][h][d] = sum_s f_s A_s[d] / sum_s f_s L_s with
// f_s = 2^(M_s - max M). grid B * nh, hd threads.
template <int NS>
__global__ __launch_bounds__(256) void k_merge(int nsplit, int hd, const float* pacc, const float* pml, float* o) {
  static_assert(NS >= 1 && NS <= 64, "one (max, sum) pair per lane");
  const int bh = blockIdx.x, d = threadIdx.x, lane = lane_id();
  const size_t base = (size_t)bh * kMaxSplit;
  // every load first: the thread's dim of each split, and split `lane`'s (max, sum) pair in lane `lane`
  float a[NS];
#pragma unroll
  for (int s2 = 0; s2 < NS; ++s2) a[s2] = pacc[(base + (size_t)min(s2, nsplit - 1)) * hd + d];
  const float2 ml = *reinterpret_cast<const float2*>(pml + (base + (size_t)min(lane, nsplit - 1)) * 2);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  const float mv = lane < nsplit ? ml.x : -INFINITY;
  float M = mv;
  M = fmaxf(M, xr_partner<32>(M));
  M = fmaxf(M, xr_partner<16>(M));
  M = fmaxf(M, xr_partner<8>(M));
  M = fmaxf(M, xr_partner<4>(M));
  M = fmaxf(M, xr_partner<2>(M));
  M = fmaxf(M, xr_partner<1>(M));
  const float f = (mv == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mv - M);  // 0 for splits past nsplit
  const float L = wave_sum(ml.y * f);
  float A = 0.f;
#pragma unroll
  for (int s2 = 0; s2 < NS; ++s2) A = fmaf(a[s2], readlane_f(f, s2), A);
  o[(size_t)bh * hd + d] = (L > 0.f) ? A / L : 0.f;
}

// ------------------------------------------------------------------------------------------------------------
}  // namespace

// ------------------------------------------------------------------------------------------------------------
// launchers

int gemm_chunks(int B, int N, int K, bool one_chunk) {
  // K chunk of 256 d (d | K / 256, d <= 4): the largest that still gives about 256 blocks
  const int q = K / 256;
  if (one_chunk) return 1;
  const int nb = ((N + 63) / 64) * ((B + 15) / 16);
  int best = q;  // chunks
  for (int d = 4; d >= 1; --d) {
    if (q % d) continue;
    best = q / d;
    if (nb * (q / d) >= 256) break;
  }
  return best;
}

hipError_t launch_gemm(hipStream_t s, int kind, int B, int N, int K, const float* X, const uint16_t* th,
                       const uint16_t* emb, const TokenSource* ts, int Bb, float escale, const uint16_t* W,
                       const uint16_t* W2, float* Y, uint16_t* Yb, int nchunks, FillRange fill, int V) {
  if (kind == 3 && (!ts || ts->k < 1 || ts->k > 64 || V < 1)) return hipErrorInvalidValue;
  if (K % 256 || N % 16 || K > kGemmMaxK || (K / 256) % nchunks) return hipErrorInvalidValue;
  const int KC = K / nchunks;
  // waves per 16-row tile: more only while the grid is below about 256 blocks (each block stages its X chunk, so
  // more blocks cost L2 reads), and at most KC / 256
  int wpt = 1;
  auto blocks = [&](int w) { return ((N + 64 / w - 1) / (64 / w)) * nchunks * ((B + 15) / 16); };
  while (wpt < 4 && wpt * 2 <= KC / 256 && blocks(wpt) < 256) wpt *= 2;
  const dim3 grid((N + 64 / wpt - 1) / (64 / wpt), nchunks, (B + 15) / 16);
  GemmSrc src{X, th, emb, ts ? *ts : TokenSource{}, V, Bb, escale};
#define MTPD_GEMM_W(KC_, WPT_, SRC_, EPI_) \
  if (KC == KC_ && wpt == WPT_) return go(k_gemm<KC_, WPT_, SRC_, EPI_>, grid, 256, 0, s, B, N, K, src, W, W2, Y, Yb, fill);
#define MTPD_GEMM(KC_, SRC_, EPI_) MTPD_GEMM_W(KC_, 1, SRC_, EPI_) MTPD_GEMM_W(KC_, 2, SRC_, EPI_) MTPD_GEMM_W(KC_, 4, SRC_, EPI_)
  if (kind == 0) {  // fp32 partials from fp32 rows
    MTPD_GEMM(256, SRC_F32, EPI_F32) MTPD_GEMM(512, SRC_F32, EPI_F32) MTPD_GEMM(768, SRC_F32, EPI_F32)
    MTPD_GEMM(1024, SRC_F32, EPI_F32)
  } else if (kind == 1) {  // bf16 out
    MTPD_GEMM(256, SRC_F32, EPI_BF16) MTPD_GEMM(512, SRC_F32, EPI_BF16) MTPD_GEMM(768, SRC_F32, EPI_BF16)
    MTPD_GEMM(1024, SRC_F32, EPI_BF16)
  } else if (kind == 2) {  // GeGLU
    MTPD_GEMM(256, SRC_F32, EPI_GEGLU) MTPD_GEMM(512, SRC_F32, EPI_GEGLU) MTPD_GEMM(768, SRC_F32, EPI_GEGLU)
    MTPD_GEMM(1024, SRC_F32, EPI_GEGLU)
  } else {  // pre_projection partials
    MTPD_GEMM(256, SRC_PRE, EPI_F32) MTPD_GEMM(512, SRC_PRE, EPI_F32) MTPD_GEMM(768, SRC_PRE, EPI_F32)
    MTPD_GEMM(1024, SRC_PRE, EPI_F32)
  }
#undef MTPD_GEMM
#undef MTPD_GEMM_W
  return hipErrorInvalidValue;
}

hipError_t launch_rownorm(hipStream_t s, int B, int H, const float* xp, int nx, size_t xs, const float* delta, int nd,
                          size_t ds, const uint16_t* w_delta, float scale, const uint16_t* w_norm, float eps,
                          float* x_new, float* u, uint64_t* keys_zero) {
  const int hpt = H / 256;
  const int NXc = nx <= 1 ? 1 : nx <= 4 ? 4 : nx <= 8 ? 8 : nx <= 16 ? 16 : 32;
  const int NDc = nd <= 1 ? 1 : nd <= 4 ? 4 : 16;
  if (H % 256 || hpt > 4 || nx > 32 || nd > 16) return hipErrorInvalidValue;
#define MTPD_RN(HPT_, NX_, ND_)                                                                                    \
  if (hpt == HPT_ && NXc == NX_ && NDc == ND_)                                                                     \
    return go(k_rownorm<HPT_, NX_, ND_>, B, 256, 0, s, B, xp, nx, xs, delta, nd, ds, w_delta, scale, w_norm, eps, \
              x_new, u, keys_zero);
#define MTPD_RN_H(NX_, ND_) MTPD_RN(1, NX_, ND_) MTPD_RN(2, NX_, ND_) MTPD_RN(3, NX_, ND_) MTPD_RN(4, NX_, ND_)
  MTPD_RN_H(1, 1) MTPD_RN_H(1, 4) MTPD_RN_H(1, 16)
  MTPD_RN_H(4, 1) MTPD_RN_H(8, 1) MTPD_RN_H(16, 1) MTPD_RN_H(32, 1)
#undef MTPD_RN_H
#undef MTPD_RN
  return hipErrorInvalidValue;
}

hipError_t launch_merge(hipStream_t s, int B, int nh, int hd, int nsplit, const float* pacc, const float* pml,
                        float* o) {
#define MTPD_MERGE(NS_) return go(k_merge<NS_>, B * nh, hd, 0, s, nsplit, hd, pacc, pml, o)
  if (nsplit <= 2) MTPD_MERGE(2);
  if (nsplit <= 4) MTPD_MERGE(4);
  if (nsplit <= 8) MTPD_MERGE(8);
  if (nsplit <= 16) MTPD_MERGE(16);
  MTPD_MERGE(32);
#undef MTPD_MERGE
}


}  // namespace mtpd
