// Dense layer kernels of the drafter step: pre_projection, q projection, o_proj (with the attention-split merge),
// GeGLU FFN, down projection, output norm + post_projection + centroid scores.
//
// Pages cited (by title; sections as headed on each page):
//   [MTP doc]    "Gemma 4 Multi-Token Prediction (MTP) drafter" (llama.cpp fork, gemma4-assistant.md)
//   [Inventory]  "Gemma 4 Assistant (MTP drafter) - tensor inventory (Stage 0)"
//   [Guide]      "Gemma 4 Assistant 使用指南：用 MTP 投机解码与 KV Sharing 加速 Gemma 4 推理" (gitcode blog)
//
//
// Dense kernels: a block owns a tile of outputs for a group of 4 batch rows; each wave computes a few outputs for
// the 4 rows with lanes striding the reduction dimension (4 elements per lane per 256-wide chunk), then a butterfly
#include "device.h"

namespace mtpd {

thread_local hipEvent_t t_ev_start = nullptr, t_ev_stop = nullptr;

namespace {

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
    asm volatile("" ::: "memory");  // all activation loads issued together (the scheduler would spread them out)
    __builtin_amdgcn_sched_barrier(0);
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
  // every load above issued here: otherwise the compiler sinks the delta-weight load into a branch on hasd and
  // waits for it there, one more dependent round trip
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
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
  const float r = rsqrt_hw(ss / (float)H + eps);
#pragma unroll
  for (int j = 0; j < NPL; ++j) xv[j] = hasd ? (xv[j] + dv[j] * r * bf2f(wd[j])) * res.scale : xv[j];
  float s2 = 0.f;
#pragma unroll
  for (int j = 0; j < NPL; ++j) s2 = fmaf(xv[j], xv[j], s2);
  s2 = wave_sum(s2);
  const float r2 = rsqrt_hw(s2 / (float)H + eps);
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
    const float f = (mv == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mv - M);
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

}  // namespace mtpd
