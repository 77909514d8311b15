// Persistent drafter kernel: n whole drafter steps (pre_projection, the Q-only decoder layers over the shared
// caches, post_projection and the centroid-masked head) for up to 16 rows in one launch, with the blocks of each XCD
// handing values to each other through that XCD's L2 instead of through kernel boundaries.
//
// Pages cited (by title; sections as headed on each page):
//   [MTP doc]    "Gemma 4 Multi-Token Prediction (MTP) drafter" (llama.cpp fork, gemma4-assistant.md)
//   [Inventory]  "Gemma 4 Assistant (MTP drafter) - tensor inventory (Stage 0)"
//   [Guide]      "Gemma 4 Assistant 使用指南：用 MTP 投机解码与 KV Sharing 加速 Gemma 4 推理" (gitcode blog)
//   [Explained]  "Gemma 4 drafter explained" (techtwitter)
//
// Shapes: hidden 256, 4 query heads of 256 over one K = V head (or two, each read by two query heads), FFN 1024,
// 2048 centroids of 128 tokens, top 32, up to 4 layers, backbone a multiple of 512 (the E2B and E4B drafters of
// [MTP doc] "Variants supported").
//
// Layout of the work. The dispatcher deals workgroups to the XCDs in turn, continuing from where the previous launch
// stopped, so block b runs on XCD (b + k) % 8 for some k of the launch. A block reads its XCD from the hardware
// XCC_ID register: it is member m = b / 8 of team t = that XCD. Team t computes rows t and t + 8 (R = 2 rows) or
// row t alone. Every block keeps the residual stream of its team's rows in LDS; a stage
// splits its outputs over the 32 members and publishes them, and the next stage polls what it needs:
//   pre     x = W_pre [hidden ; escale E[token]]      8 outputs per member, K split over the 4 waves
//   q       q = W_q RMSNorm(x; attn_norm)             32 outputs per member
//   att     q_norm + RoPE, flash-decode partials      keys of a row split over the 16 (R = 2) or 32 members
//   mrg     log-sum-exp merge of the partials         64 (32) dims per member
//   op      W_o o                                     8 outputs per member, K split over the waves
//   ffn     gelu(W_g u) * (W_u u), u = RMSNorm(x + RMSNorm(W_o o; post_attn); ffn_norm)   32 per member
//   dn      W_d m                                     8 outputs per member
//   post    h = RMSNorm(x; output_norm); W_post h (bf16), centroids . h
//   head    top-32 of the row's 2048 scores (every member, redundantly), the member's 2 (1) slots: ids, sparse
//           logits, scatter into the -1e30 row, the slot's best (value, id) key
// The next step's pre takes the row's token as the best of the 32 slot keys.
//
// Exchange words: bits 0-31 the payload (an fp32, or two bf16), bits 32-63 the tag (launch epoch + step + 1) * 32
// + stage id. A producer stores the word into its XCD's L2 (a workgroup-scope store: written through the CU's L1);
// a consumer loads with device-scope loads, which skip the L1 and read the L2, until every word it needs carries the
// expected tag. Tags never repeat, so stale words from earlier stages, steps or launches are simply not accepted,
// and no buffer is ever cleared. A word's slot is rewritten only after every consumer of its previous value has
// published something the writer waited for, so no value is overwritten before it is read.
// The two widest hand-offs (the merged attention output, 2048 values of which every member reads 2048, and the
// centroid scores) go out as untagged fp32 values instead: the producing wave waits until its stores have reached L2
// (vmcnt(0)) and then stores one tagged flag word; a consumer spins on the few flags of the producers it needs and
// then reads the values once. Re-reading 2048 tagged words on every spin costs more than the extra round trip.
#include "attn_mfma.h"

namespace mtpd {
namespace {

constexpr int TM = 32;     // members per team (CUs per XCD)
constexpr int NT = 8;      // teams (XCDs)
constexpr int TH = 256;    // drafter width
constexpr int TQ = 1024;   // query heads x head_dim
constexpr int TF = 1024;   // FFN width
constexpr int TC = 2048;   // centroids
constexpr int TKS = 32;    // clusters kept
constexpr int TVS = 128;   // tokens per cluster
constexpr int NSID = 32;   // stage ids per step
constexpr int kSpin = 1 << 18;  // polls before a wait gives up (far beyond any real wait)

// stage ids
constexpr int S_PRE = 0;
__device__ __forceinline__ int s_q(int l) { return 1 + 6 * l; }
__device__ __forceinline__ int s_att(int l) { return 2 + 6 * l; }
__device__ __forceinline__ int s_mrg(int l) { return 3 + 6 * l; }
__device__ __forceinline__ int s_op(int l) { return 4 + 6 * l; }
__device__ __forceinline__ int s_ffn(int l) { return 5 + 6 * l; }
__device__ __forceinline__ int s_dn(int l) { return 6 + 6 * l; }
constexpr int S_POST = 25, S_KEY = 26;

// exchange regions of one team (64-bit words)
constexpr int AP_STRIDE = 4 * 258;  // per member: 4 heads x (256 partial sums, max, sum)
constexpr int A_XB = 0;
constexpr int A_Q = A_XB + 2 * TH;
constexpr int A_AP = A_Q + 2 * TQ;
constexpr int A_O = A_AP + TM * AP_STRIDE;  // untagged fp32 pairs, announced by the A_OFL flags
constexpr int A_T = A_O + 2 * TQ;
constexpr int A_M = A_T + 2 * TH;
constexpr int A_D = A_M + 2 * TF;
constexpr int A_HID = A_D + 2 * TH;        // 2 rows x up to 2048 words (bf16 pairs of a 4096-wide hidden)
constexpr int A_SC = A_HID + 2 * 2048;    // untagged fp32 centroid scores, announced by the A_SFL flags
constexpr int A_KEY = A_SC + 2 * TC;       // 2 rows x 32 slots x (low, high) halves of the (value, id) key
constexpr int A_OFL = A_KEY + 2 * TKS * 2;  // flags of the merged attention output (one per member)
constexpr int A_SFL = A_OFL + TM;           // flags of the centroid scores (one per wave of every member)
constexpr int A_END = A_SFL + 4 * TM;
constexpr int TEAM_WORDS = (A_END + 511) & ~511;

// packed dense weights (bf16 elements): kTeamMaxLayers layers of [q | q_norm | o | attn_norm | post_attn_norm |
// ffn_norm | post_ffw_norm | gate | up | down], then pre_proj [256][2 Bb], post_proj [Bb][256], output_norm,
// centroids [2048][256]
constexpr size_t W_Q = 0;
constexpr size_t W_QN = W_Q + (size_t)TQ * TH;
constexpr size_t W_O = W_QN + 256;
constexpr size_t W_AN = W_O + (size_t)TH * TQ;
constexpr size_t W_PAN = W_AN + TH;
constexpr size_t W_FN = W_PAN + TH;
constexpr size_t W_PFN = W_FN + TH;
constexpr size_t W_G = W_PFN + TH;
constexpr size_t W_U = W_G + (size_t)TF * TH;
constexpr size_t W_D = W_U + (size_t)TF * TH;
constexpr size_t W_LAYER = W_D + (size_t)TH * TF;
constexpr size_t W_PRE = (size_t)kTeamMaxLayers * W_LAYER;
__host__ __device__ constexpr size_t w_post(int Bb) { return W_PRE + (size_t)TH * 2 * Bb; }
__host__ __device__ constexpr size_t w_onorm(int Bb) { return w_post(Bb) + (size_t)Bb * TH; }
__host__ __device__ constexpr size_t w_cen(int Bb) { return w_onorm(Bb) + TH; }
__host__ __device__ constexpr size_t w_total(int Bb) { return w_cen(Bb) + (size_t)TC * TH; }
__device__ __forceinline__ const uint16_t* lw(const TeamArgs& a, int l, size_t off) {
  return a.wpk + (size_t)l * W_LAYER + off;
}

// Stage timeline for measurement builds (-DMTPD_TEAM_TRACE): thread 0 of every block records the wall clock
// (100 MHz) when the block enters each stage (entry step * 64 + stage id) and at points inside some stages
// (entries 32 and up).
#ifdef MTPD_TEAM_TRACE
__device__ uint64_t g_team_trace[256 * 256];
#define TEAM_TRACE(step, sid)                                                                            \
  do {                                                                                                   \
    if (threadIdx.x == 0 && (step) < 4) g_team_trace[blockIdx.x * 256 + (step) * 64 + (sid)] = wall_clock64(); \
  } while (0)
#define TEAM_TRACE_AT(step, sid, thread)                                                                 \
  do {                                                                                                   \
    if (threadIdx.x == (thread) && (step) < 4) g_team_trace[blockIdx.x * 256 + (step) * 64 + (sid)] = wall_clock64(); \
  } while (0)
// the shader cycle counter instead of the wall clock (the two give the shader clock rate)
#define TEAM_TRACE_CYCLES(step, sid)                                                                         \
  do {                                                                                                       \
    if (threadIdx.x == 0 && (step) < 4) g_team_trace[blockIdx.x * 256 + (step) * 64 + (sid)] = clock64(); \
  } while (0)
// the same after the value v is computed (an empty asm that consumes it keeps the clock read behind it)
#define TEAM_TRACE_DEP(step, sid, v)              \
  do {                                            \
    const float tdv_ = (v);                       \
    asm volatile("" ::"v"(tdv_) : "memory");      \
    TEAM_TRACE(step, sid);                        \
  } while (0)
#else
#define TEAM_TRACE_CYCLES(step, sid) \
  do {                               \
  } while (0)
#define TEAM_TRACE_DEP(step, sid, v) \
  do {                               \
  } while (0)
#define TEAM_TRACE_AT(step, sid, thread) \
  do {                                   \
  } while (0)
#define TEAM_TRACE(step, sid) \
  do {                        \
  } while (0)
#endif

__device__ __forceinline__ void put(uint64_t* p, uint32_t tag, uint32_t bits) {
  __hip_atomic_store(p, ((uint64_t)tag << 32) | bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void putf(uint64_t* p, uint32_t tag, float v) { put(p, tag, __float_as_uint(v)); }
__device__ __forceinline__ uint64_t peek(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

struct Team {
  int t, m, R;           // team, member, rows of the team
  int row0, row1;        // batch rows
  __device__ __forceinline__ int row(int r) const { return r ? row1 : row0; }
  uint32_t E;            // this launch's epoch (steps before it)
  uint64_t* X;           // the team's exchange words
  uint32_t* status;
  bool dead;             // a wait of this wave ran out: later waits return at once
  // (+1: the arena starts zeroed, so tag 0 must never be waited for)
  __device__ __forceinline__ uint32_t tag(int step, int sid) const { return (E + (uint32_t)step + 1u) * NSID + (uint32_t)sid; }
};

// Wave-wide wait: lane loads N words X[idx[j]] until every word of every lane carries `tag`; the payloads land in
// out. All N loads are issued together on every poll.
template <int N>
__device__ __forceinline__ void wait_words(Team& T, const int (&idx)[N], uint32_t tag, int sid, uint32_t (&out)[N]) {
  uint64_t v[N];
  int spin = 0;
  for (;;) {
#pragma unroll
    for (int j = 0; j < N; ++j) v[j] = peek(T.X + idx[j]);
    bool ok = true;
#pragma unroll
    for (int j = 0; j < N; ++j) ok = ok && ((uint32_t)(v[j] >> 32) == tag);
    if (__all(ok) || T.dead) break;
    if (++spin >= kSpin) {
      T.dead = true;
      if (lane_id() == 0) {
        __hip_atomic_fetch_or(T.status, kTeamTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        // one plus the stage id, made opaque here so that the compiler does not keep the constant in a register
        // across the whole launch for this rarely taken path
        uint32_t st = (uint32_t)sid + 1u;
        asm volatile("" : "+v"(st));
        __hip_atomic_fetch_max(T.status + 1, st, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      break;
    }
  }
#pragma unroll
  for (int j = 0; j < N; ++j) out[j] = (uint32_t)v[j];
}

struct Smem {
  float xs[2][TH];   // residual stream of the team's rows
  float us[2][TH];   // normed input of the current stage (the head's h after post)
  float red[4][64];  // cross-wave partial sums
  float mrgl[4];
  int tok[2];
  // attention
  // [step][hi/lo][head slot][kq][8 dims]; slots 4 .. 7 stay zero (unused columns of the score tile)
  __attribute__((aligned(16))) uint16_t qop[8][2][8][4][8];
  // q staging, then the waves' combine tiles: [wave][dim][hi rows of heads 0..3 | lo rows of heads 0..3]
  __attribute__((aligned(16))) float qs_wacc[4 * 256 * 8];
  __attribute__((aligned(16))) uint16_t vt[4][16][264];
  __attribute__((aligned(16))) float wml[4][4][2];
  // this member's split of its row's sliding window, resident for the whole launch (every sliding layer of every
  // step reads the same keys): up to 64 keys of 256 dims, rows padded like the V tiles
  __attribute__((aligned(16))) uint16_t ks[64][264];
  // head
  uint64_t cand[TC];
  int sel[TKS];
  uint32_t ncand;
  uint32_t wtot[4];
  uint64_t bestw[2][4];
};

template <int R>
constexpr int kRedLanes = 64 / (R * 8);  // lanes per value after XR<R*8, 32>

// Residual update and norm of one row in one wave (dims 64 e + lane): xs[r] <- f(xs[r], delta), us[r] <- RMSNorm.
// mode 0: x = delta (pre_projection output); 1: x = (x + RMSNorm(delta; wd)) * sc; 2: x = x + RMSNorm(delta; wd).
__device__ __forceinline__ void row_update(Smem& S, int r, int mode, const float (&delta)[4], const uint16_t (&wd)[4],
                                           float sc, const uint16_t (&wn)[4], float eps) {
  const int lane = lane_id();
  float xv[4];
  if (mode == 0) {
#pragma unroll
    for (int e = 0; e < 4; ++e) xv[e] = delta[e];
  } else {
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) ss = fmaf(delta[e], delta[e], ss);
    ss = wave_sum(ss);
    const float rr = rsqrt_hw(ss / (float)TH + eps);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float v = S.xs[r][64 * e + lane] + delta[e] * rr * bf2f(wd[e]);
      xv[e] = (mode == 1) ? v * sc : v;
    }
  }
  float s2 = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) s2 = fmaf(xv[e], xv[e], s2);
  s2 = wave_sum(s2);
  const float r2 = rsqrt_hw(s2 / (float)TH + eps);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    S.xs[r][64 * e + lane] = xv[e];
    S.us[r][64 * e + lane] = xv[e] * r2 * bf2f(wn[e]);
  }
}

// Poll one 256-wide row region (dims 64 e + lane) of the exchange into delta.
__device__ __forceinline__ void poll_row(Team& T, int off, uint32_t tag, int sid, float (&delta)[4]) {
  const int lane = lane_id();
  int idx[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) idx[e] = off + 64 * e + lane;
  uint32_t raw[4];
  wait_words<4>(T, idx, tag, sid, raw);
#pragma unroll
  for (int e = 0; e < 4; ++e) delta[e] = __uint_as_float(raw[e]);
}

__device__ __forceinline__ void load_w4(const uint16_t* w, uint16_t (&out)[4]) {
  const int lane = lane_id();
#pragma unroll
  for (int e = 0; e < 4; ++e) out[e] = w[64 * e + lane];
}

__device__ __forceinline__ float dot4(uint2 w, float4 u) {
  float wf[4];
  unpack4(w, wf);
  return fmaf(u.x, wf[0], fmaf(u.y, wf[1], fmaf(u.z, wf[2], u.w * wf[3])));
}

// ------------------------------------------------------------------------------------------------------------
// Each stage's weight slices are requested one stage ahead: a stage issues the next stage's loads as soon as its
// own inputs have arrived, so their latency overlaps its arithmetic and the next exchange instead of gating the
// next poll (a wait covers every load issued before the one it needs).

template <int NBB>
struct WPre {
  uint2 w[8][NBB / 2];
};
struct WQ {
  uint2 w[8];
  uint16_t an[4], pfn[4];  // attn_norm of the layer, post_ffw_norm of the previous layer
};
struct WK {
  uint2 w[8];  // o_proj or down: 8 outputs over this wave's quarter of K = 1024
};
struct WF {
  uint2 g[8], u[8];
  uint16_t fn[4], pan[4];  // ffn_norm, post_attention_norm
};
template <int NBB>
struct WPost {
  uint2 p[((NBB * 2 + 7) / 8) * 8], c[16];
  uint16_t on[4], pfn[4];  // output_norm, the last layer's post_ffw_norm
};

template <int NBB>
__device__ __forceinline__ void issue_pre(const TeamArgs& a, const Team& T, WPre<NBB>& W) {
  constexpr int Bb = NBB * 256, CPL = NBB / 2;
  const int w = wave_id(), lane = lane_id(), n0 = 8 * T.m, kb = w * (Bb / 2);
#pragma unroll
  for (int o = 0; o < 8; ++o)
#pragma unroll
    for (int c = 0; c < CPL; ++c)
      W.w[o][c] = *reinterpret_cast<const uint2*>(a.wpk + W_PRE + (size_t)(n0 + o) * (2 * Bb) + kb + 256 * c + 4 * lane);
}

__device__ __forceinline__ void issue_q(const TeamArgs& a, const Team& T, int l, WQ& W) {
  const int w = wave_id(), lane = lane_id(), n0 = 32 * T.m + 8 * w;
#pragma unroll
  for (int o = 0; o < 8; ++o) W.w[o] = *reinterpret_cast<const uint2*>(lw(a, l, W_Q) + (size_t)(n0 + o) * TH + 4 * lane);
  load_w4(lw(a, l, W_AN), W.an);
  load_w4(lw(a, l > 0 ? l - 1 : 0, W_PFN), W.pfn);
}

__device__ __forceinline__ void issue_k1024(const uint16_t* Wm, const Team& T, WK& W) {
  const int w = wave_id(), lane = lane_id(), n0 = 8 * T.m, k = 256 * w + 4 * lane;
#pragma unroll
  for (int o = 0; o < 8; ++o) W.w[o] = *reinterpret_cast<const uint2*>(Wm + (size_t)(n0 + o) * 1024 + k);
}

__device__ __forceinline__ void issue_ffn(const TeamArgs& a, const Team& T, int l, WF& W) {
  const int w = wave_id(), lane = lane_id(), f0 = 32 * T.m + 8 * w;
#pragma unroll
  for (int o = 0; o < 8; ++o) {
    W.g[o] = *reinterpret_cast<const uint2*>(lw(a, l, W_G) + (size_t)(f0 + o) * TH + 4 * lane);
    W.u[o] = *reinterpret_cast<const uint2*>(lw(a, l, W_U) + (size_t)(f0 + o) * TH + 4 * lane);
  }
  load_w4(lw(a, l, W_FN), W.fn);
  load_w4(lw(a, l, W_PAN), W.pan);
}

// the centroid rows and norms of the post stage (before its poll: the head waits for the scores)
template <int NBB>
__device__ __forceinline__ void issue_post_cen(const TeamArgs& a, const Team& T, WPost<NBB>& W) {
  constexpr int Bb = NBB * 256;
  const int w = wave_id(), lane = lane_id();
  const int c0 = 64 * T.m + 16 * w;
#pragma unroll
  for (int o = 0; o < 16; ++o) W.c[o] = *reinterpret_cast<const uint2*>(a.wpk + w_cen(Bb) + (size_t)(c0 + o) * TH + 4 * lane);
  load_w4(a.wpk + w_onorm(Bb), W.on);
  load_w4(lw(a, a.n_layer - 1, W_PFN), W.pfn);
}

// the post_projection rows (after the poll: only the next step's pre reads their outputs)
template <int NBB>
__device__ __forceinline__ void issue_post_proj(const TeamArgs& a, const Team& T, WPost<NBB>& W) {
  constexpr int Bb = NBB * 256, NPB = Bb / 32, NPW = NPB / 4, NPG = (NPW + 7) / 8;
  const int w = wave_id(), lane = lane_id();
  const int p0 = NPB * T.m + NPW * w;
#pragma unroll
  for (int o = 0; o < NPG * 8; ++o)
    W.p[o] = *reinterpret_cast<const uint2*>(a.wpk + w_post(Bb) + (size_t)(p0 + min(o, NPW - 1)) * TH + 4 * lane);
}

// Part p of np of this member's 1/32 of the step's -1e30 base rows ([Inventory] "Centroid / ordered embeddings LM
// head", step 5), as streaming stores of waves 2 and 3. The q and ffn stages issue it right after their own
// publishes (stores issued before a publish hold the published words back), so the 16 MB of each step's fill spreads
// over the layers and drains while the next stage waits; every wave passes a full wait before it publishes the
// centroid scores the head waits for, so the fill precedes every scatter.
template <int R>
__device__ __forceinline__ void fill_part(const TeamArgs& a, const Team& T, int step, int p, int np) {
  if (!a.logits || wave_id() < 2) return;
  const size_t V = (size_t)a.V;
  const size_t per = ((V + TM - 1) / TM + 3) & ~(size_t)3;
  const size_t b0 = (size_t)T.m * per;
  const size_t e0 = b0 + per < V ? b0 + per : V;
  const size_t q = ((per + np - 1) / np + 3) & ~(size_t)3;
  const size_t s0 = b0 + (size_t)p * q;
  const size_t s1 = (p == np - 1) ? e0 : (s0 + q < e0 ? s0 + q : e0);
  const f32x4 neg = f32x4{-1e30f, -1e30f, -1e30f, -1e30f};
  const int tt = threadIdx.x - 128;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    float* rowp = a.logits + ((size_t)step * a.B + T.row(r)) * V;
    for (size_t i = s0 + 4 * (size_t)tt; i + 4 <= s1; i += 512)
      __builtin_nontemporal_store(neg, reinterpret_cast<f32x4*>(rowp + i));
  }
}

// ------------------------------------------------------------------------------------------------------------
// pre_projection of [hidden ; escale E[token]] ([MTP doc] "What it is": 2x backbone input; [Guide] section 2(3);
// [Explained] "Target Activations"). Member m: outputs 8m .. 8m + 7. Wave w covers K quarter w: waves 0-1 the
// hidden half, waves 2-3 the embedding half (Bb % 512 == 0: NBB / 2 chunks of 4 elements per lane).

template <int R, int NBB, int NKV>
__device__ __forceinline__ void stage_pre(const TeamArgs& a, Team& T, Smem& S, int step, WQ& Wq,
                                          const uint32_t (&pf)[2]) {
  WPre<NBB> W;
  // the hidden half's slices now; the embedding half's after the key wait below, so that the wait does not also
  // cover these loads (loads complete in order)
  if (wave_id() < 2) issue_pre<NBB>(a, T, W);
  constexpr int Bb = NBB * 256, CPL = NBB / 2;
  const int w = wave_id(), lane = lane_id();
  const int n0 = 8 * T.m;
  const int kb = w * (Bb / 2);  // first element of this wave's quarter of K = 2 Bb
  // step 0 also brings in this member's split of the sliding window (the split of stage_att), which stays in S.ks
  // for the whole launch: every sliding layer of every step reads the same keys. 8 rows of 512 bytes per pass; with
  // two kv heads, rows 0 .. 31 hold kv head 0's keys of the split and rows 32 .. 63 kv head 1's.
  uint4 kres[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) kres[i] = make_uint4(0u, 0u, 0u, 0u);
  if (step == 0) {
    constexpr int NS = TM / R;
    const int r = (R == 2) ? (T.m >> 4) : 0, sp = (R == 2) ? (T.m & 15) : T.m, row = T.row(r);
    const int cnt = a.win_count[0][row], start = a.win_start[0][row], cap = a.cap[0];
    const int chunk = (cnt + NS - 1) / NS;
    const int k0 = start + sp * chunk, k1 = min(start + cnt, k0 + chunk);
    constexpr bool two = NKV == 2;
    const uint16_t* Kb = a.kc[0] + (size_t)row * NKV * cap * 256;
    const uint16_t* Kb1 = two ? Kb + (size_t)cap * 256 : Kb;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      // passes 4 .. 7 (rows 32 .. 63) take kv head 1's keys from the split's start when there are two
      const bool g1 = i >= 4 && two;
      const int t = max(min(k0 + (threadIdx.x >> 5) + 8 * (g1 ? i - 4 : i), k1 - 1), start);
      kres[i] = *reinterpret_cast<const uint4*>((g1 ? Kb1 : Kb) + (size_t)slot_of(t, cap) * 256 +
                                                (threadIdx.x & 31) * 8);
    }
  }
  uint2 xr[R][CPL];
  const bool emb = w >= 2;
  if (!emb) {
    if (step == 0) {
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int c = 0; c < CPL; ++c)
          xr[r][c] = *reinterpret_cast<const uint2*>(a.th + (size_t)T.row(r) * Bb + kb + 256 * c + 4 * lane);
    } else {
      int idx[R * CPL * 2];
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          const int k = kb + 256 * c + 4 * lane;  // even: bf16 pairs (k, k+1) and (k+2, k+3)
          idx[(r * CPL + c) * 2] = A_HID + r * 2048 + k / 2;
          idx[(r * CPL + c) * 2 + 1] = A_HID + r * 2048 + k / 2 + 1;
        }
      uint32_t raw[R * CPL * 2];
      wait_words<R * CPL * 2>(T, idx, T.tag(step - 1, S_POST), S_POST, raw);
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int c = 0; c < CPL; ++c) xr[r][c] = make_uint2(raw[(r * CPL + c) * 2], raw[(r * CPL + c) * 2 + 1]);
    }
    asm volatile("" ::"v"(pf[0]), "v"(pf[1]));  // the previous head's row touches end here
    issue_q(a, T, 0, Wq);
  } else {
    // the row's token: the caller's at step 0, else the best of the previous step's 32 slot keys
    int tk[R];
    if (step == 0) {
#pragma unroll
      for (int r = 0; r < R; ++r) tk[r] = a.tok[T.row(r)];
    } else {
      int idx[R];
#pragma unroll
      for (int r = 0; r < R; ++r) idx[r] = A_KEY + r * (2 * TKS) + lane;  // lane = 2 slot + half
      uint32_t raw[R];
      wait_words<R>(T, idx, T.tag(step - 1, S_KEY), S_KEY, raw);
      TEAM_TRACE_AT(step, 44, 128);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const uint32_t lo = pair_lane<0>(raw[r]), hi = pair_lane<1>(raw[r]);
        tk[r] = key_id(wave_max_u64(((uint64_t)hi << 32) | lo));
        if (w == 2 && lane == 0 && T.m == 0 && a.tokens)
          a.tokens[(size_t)T.row(r) * a.tok_stride + (step - 1)] = tk[r];
      }
    }
    issue_pre<NBB>(a, T, W);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int t = tk[r] < 0 ? 0 : (tk[r] >= a.V ? a.V - 1 : tk[r]);  // out-of-range ids are clamped
#pragma unroll
      for (int c = 0; c < CPL; ++c)
        xr[r][c] = *reinterpret_cast<const uint2*>(a.temb + (size_t)t * Bb + (kb - Bb) + 256 * c + 4 * lane);
    }
    issue_q(a, T, 0, Wq);
  }
  // both operands are bf16 (weights, the hidden state or embedding row), so pairs go through the packed bf16 dot
  // with fp32 accumulation; the embedding scale multiplies the wave's sums
  const float sc = emb ? a.escale : 1.0f;
  float acc[R * 8];
#pragma unroll
  for (int i = 0; i < R * 8; ++i) acc[i] = 0.f;
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int c = 0; c < CPL; ++c)
#pragma unroll
      for (int o = 0; o < 8; ++o) {
        float s = acc[r * 8 + o];
        s = dot2_bf16(xr[r][c].x, W.w[o][c].x, s);
        s = dot2_bf16(xr[r][c].y, W.w[o][c].y, s);
        acc[r * 8 + o] = s;
      }
#pragma unroll
  for (int i = 0; i < R * 8; ++i) acc[i] *= sc;
  TEAM_TRACE_AT(step, 45, 128);
  XR<R * 8, 32>::run(acc, lane);
  constexpr int RL = kRedLanes<R>;
  if (lane % RL == 0) S.red[w][lane / RL] = acc[0];
  if (step == 0) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      *reinterpret_cast<uint4*>(&S.ks[(threadIdx.x >> 5) + 8 * i][(threadIdx.x & 31) * 8]) = kres[i];
  }
  __syncthreads();
  TEAM_TRACE(step, 46);
  if (threadIdx.x < R * 8) {
    const int i = threadIdx.x;
    const float v = S.red[0][i] + S.red[1][i] + S.red[2][i] + S.red[3][i];
    putf(T.X + A_XB + (i >> 3) * TH + n0 + (i & 7), T.tag(step, S_PRE), v);
  }
  __syncthreads();
}

// ------------------------------------------------------------------------------------------------------------
// q projection ([MTP doc] "Tensor schema": attn_norm, attn_q). Layer 0 takes the pre_projection output as the
// residual stream; later layers first finish the previous layer's FFN residual:
// x = (x + RMSNorm(W_d m; post_ffw_norm)) * layer_output_scale ([MTP doc] "What it is": per-layer scalar).

// This member's split of a row's key window in the attention stage of layer l (stage_att's layout).
struct KeySplit {
  const uint16_t* Kb;  // the row's cache of kv head 0, + 8 kq
  int k0, k1, start, cap;
  int nbg;  // 64-key rounds per kv head (two kv heads: batches nbg .. 2 nbg - 1 read kv head 1)
};

template <int R, int NKV>
__device__ __forceinline__ KeySplit key_split(const TeamArgs& a, const Team& T, int type) {
  constexpr int NS = TM / R;
  const int kq = lane_id() >> 4;
  const int r = (R == 2) ? (T.m >> 4) : 0, s = (R == 2) ? (T.m & 15) : T.m;
  const int row = T.row(r);
  KeySplit k;
  const int cnt = a.win_count[type][row];
  k.start = a.win_start[type][row];
  k.cap = a.cap[type];
  const int chunk = (cnt + NS - 1) / NS;
  k.k0 = k.start + s * chunk;
  k.k1 = min(k.start + cnt, k.k0 + chunk);
  k.Kb = a.kc[type] + (size_t)row * NKV * k.cap * 256 + 8 * kq;
  k.nbg = (k.k1 - k.k0 + 63) / 64;
  return k;
}

// Batch j of this wave in a streamed split: keys k0 + 64 j' + 16 w .. +16 of kv head g, where j = g nbg + j' (rows
// past the split clamped to its last key: cache hits, masked in the scores).
template <int NKV>
__device__ __forceinline__ void load_key_batch(const KeySplit& k, int j, uint4 (&dst)[8]) {
  const int g = (NKV == 2 && j >= k.nbg) ? 1 : 0;
  const int tt = k.k0 + 64 * (j - g * k.nbg) + 16 * wave_id() + (lane_id() & 15);
  const uint16_t* rp = k.Kb + ((size_t)g * k.cap + slot_of(max(min(tt, k.k1 - 1), k.start), k.cap)) * 256;
#pragma unroll
  for (int c = 0; c < 8; ++c) dst[c] = *reinterpret_cast<const uint4*>(rp + 32 * c);
}

template <int R>
__device__ __forceinline__ void stage_q(const TeamArgs& a, Team& T, Smem& S, int step, int l, const WQ& W) {
  const int w = wave_id(), lane = lane_id();
  const int n0 = 32 * T.m + 8 * w;
  const int lp = l > 0 ? l - 1 : 0;
  if (w < R) {
    float d[4];
    if (l == 0)
      poll_row(T, A_XB + w * TH, T.tag(step, S_PRE), S_PRE, d);
    else
      poll_row(T, A_D + w * TH, T.tag(step, s_dn(l - 1)), s_dn(l - 1), d);
    if (l == 1) TEAM_TRACE(step, 32);
    row_update(S, w, l == 0 ? 0 : 1, d, W.pfn, a.scale[lp], W.an, a.eps);
  }
  __syncthreads();
  float acc[R * 8];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const float4 u = *reinterpret_cast<const float4*>(&S.us[r][4 * lane]);
#pragma unroll
    for (int o = 0; o < 8; ++o) acc[r * 8 + o] = dot4(W.w[o], u);
  }
  XR<R * 8, 32>::run(acc, lane);
  constexpr int RL = kRedLanes<R>;
  if (lane % RL == 0) {
    const int i = lane / RL;
    putf(T.X + A_Q + (i >> 3) * TQ + n0 + (i & 7), T.tag(step, s_q(l)), acc[0]);
  }
  fill_part<R>(a, T, step, 2 * l, 2 * a.n_layer);  // behind the publish, so it does not delay the q words
}

// ------------------------------------------------------------------------------------------------------------
// Shared-cache attention ([MTP doc] "What it is": Q-only attention over the target's last-layer K/V of the layer's
// type; [Guide] section 2(4): one query, the sliding mask keeps the last `window` keys, the full layer every key;
// [Inventory] "Notes for llama.cpp port" 2: V = K). q_norm + rotation at the row's constant position ([Guide]
// section 2(2)). Member m takes split s of its row's key window; wave w normalises and rotates head w.

template <int R, int NKV>
__device__ __forceinline__ void stage_att(const TeamArgs& a, Team& T, Smem& S, int step, int l, WK& Wo) {
  constexpr int HD = 256, KSTEPS = 8, TILES = 16, NS = TM / R, half = HD / 2;
  const int w = wave_id(), lane = lane_id();
  const int hq = lane & 15, kq = lane >> 4;
  const int type = (a.full_mask >> l) & 1u;
  const int r = (R == 2) ? (T.m >> 4) : 0, s = (R == 2) ? (T.m & 15) : T.m;
  const int row = T.row(r);
  const int cnt = a.win_count[type][row], start = a.win_start[type][row], cap = a.cap[type];
  const int chunk = (cnt + NS - 1) / NS;
  const int k0 = start + s * chunk;
  const int k1 = min(start + cnt, k0 + chunk);
  const uint16_t* Kb = a.kc[type] + (size_t)row * NKV * cap * HD + 8 * kq;
  constexpr bool two = NKV == 2;
  // the split sits in S.ks (loaded at the start of the launch)
  const bool resident = type == 0 && chunk <= (two ? 32 : 64);
  // inputs of q_norm + rotation, then the first key batch: none of them waits on the q projection
  const float* tab = a.rope + ((size_t)row * 2 + type) * 2 * half;
  const uint2 qw = *reinterpret_cast<const uint2*>(lw(a, l, W_QN) + lane * 4);
  const int i0 = (lane * 4) & (half - 1);
  const float4 co4 = *reinterpret_cast<const float4*>(tab + i0);
  const float4 si4 = *reinterpret_cast<const float4*>(tab + half + i0);
  // streamed splits keep three 16-key batches of this wave in flight
  const KeySplit ksp = key_split<R, NKV>(a, T, type);
  uint4 kA[KSTEPS], kB[KSTEPS], kC[KSTEPS];
  if (!resident) {
    load_key_batch<NKV>(ksp, 0, kA);
    load_key_batch<NKV>(ksp, 1, kB);
    load_key_batch<NKV>(ksp, 2, kC);
  }
  // q of head w (dims 4 lane .. +3), whose rotation partners (d <-> d + 128) sit in lane ^ 32
  float v[4];
  {
    int idx[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) idx[e] = A_Q + r * TQ + w * HD + 4 * lane + e;
    uint32_t raw[4];
    wait_words<4>(T, idx, T.tag(step, s_q(l)), s_q(l), raw);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = __uint_as_float(raw[e]);
  }
  // the o_proj slice, used two stages on: requested only now, so that the q poll above does not wait for it
  issue_k1024(lw(a, l, W_O), T, Wo);
  if (type) TEAM_TRACE(step, 28);
  if (l == 1) TEAM_TRACE(step, 33);
  {
    float wq[4];
    unpack4(qw, wq);
    const float co[4] = {co4.x, co4.y, co4.z, co4.w}, si[4] = {si4.x, si4.y, si4.z, si4.w};
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) ss = fmaf(v[e], v[e], ss);
    ss = wave_sum(ss);
    const float rr = rsqrt_hw(ss / (float)HD + a.eps);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = v[e] * rr * wq[e];
    // the rotated q goes straight into the score operand: dims 4 lane .. +3 of head w are step c = lane / 8,
    // kq = (lane % 8) / 2, elements 4 (lane % 2) .. +3, as a bf16 hi part and the bf16 rest
    float qv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float partner = xr_partner<32>(v[e]);
      qv[e] = (lane < 32) ? (v[e] * co[e] - partner * si[e]) : (v[e] * co[e] + partner * si[e]);
    }
    uint16_t hb[4], lb[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      hb[e] = f2bf(qv[e]);
      lb[e] = f2bf(qv[e] - bf2f(hb[e]));
    }
    const int c = lane >> 3, kk = (lane & 7) >> 1, e0 = 4 * (lane & 1);
    *reinterpret_cast<uint2*>(&S.qop[c][0][w][kk][e0]) =
        make_uint2((uint32_t)hb[0] | ((uint32_t)hb[1] << 16), (uint32_t)hb[2] | ((uint32_t)hb[3] << 16));
    *reinterpret_cast<uint2*>(&S.qop[c][1][w][kk][e0]) =
        make_uint2((uint32_t)lb[0] | ((uint32_t)lb[1] << 16), (uint32_t)lb[2] | ((uint32_t)lb[3] << 16));
  }
  if (l == 1) TEAM_TRACE(step, 47);
  __syncthreads();
  if (l == 1) TEAM_TRACE(step, 48);
  if (type) TEAM_TRACE(step, 29);
  if (l == 1) TEAM_TRACE(step, 49);
  float mrun = -INFINITY, lrun = 0.f;
  if (resident) {
    // every wave scores all of the split's keys and accumulates P.V for dims 64 w .. 64 w + 63, so the member's
    // partial is complete in each wave's quarter of the dims and goes out without a combine
    f32x4 acc4[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) acc4[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    // rows 16 j .. 16 j + 31 of S.ks: keys k0 + 16 j .. of the one kv head, or (two kv heads) keys k0 .. k0 + 31
    // of kv head j / 2, which only its query heads j .. j + 1 read
#pragma unroll
    for (int j = 0; j < 4; j += 2) {
      const int tb = two ? k0 : k0 + 16 * j;
      if (tb < k1) {  // block-uniform
        uint4 kk[2][KSTEPS];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int c = 0; c < KSTEPS; ++c)
            kk[i][c] = *reinterpret_cast<const uint4*>(&S.ks[16 * (j + i) + hq][32 * c + 8 * kq]);
        mfma_tiles2_dims(tb, k1, a.scale_log2, &S.ks[16 * j][0], S.qop, kk, w, acc4, mrun, lrun, two ? j : 0,
                         two ? j + 2 : 4);
      }
    }
    if (l == 1) TEAM_TRACE(step, 50);
    // rows 8 .. 11 (lo products) join rows 0 .. 3 (hi) in lanes 32 apart; lanes of kq 0 then publish tiles 0 and 1,
    // lanes of kq 2 tiles 2 and 3
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc4[t][r] += xr_partner<32>(acc4[t][r]);
    const uint32_t tg = T.tag(step, s_att(l));
    uint64_t* ap = T.X + A_AP + T.m * AP_STRIDE;
    if (kq == 0 || kq == 2) {
      const int tp = kq >> 1;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int d = 64 * w + 16 * (2 * tp + i) + hq;
#pragma unroll
        for (int hh = 0; hh < 4; ++hh) putf(ap + hh * 258 + d, tg, tp ? acc4[2 + i][hh] : acc4[i][hh]);
      }
    }
    if (w == 0 && lane < 4) {  // head `lane`: its running maximum and sum (the same in every wave)
      putf(ap + lane * 258 + 256, tg, mrun);
      putf(ap + lane * 258 + 257, tg, lrun);
    }
    return;
  }
  f32x4 acc[TILES];
#pragma unroll
  for (int t = 0; t < TILES; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  uint16_t* tile = &S.vt[w][0][0];
  // 64-key rounds of the block (one 16-key batch per wave each); with two kv heads, rounds nb .. 2 nb - 1 take kv
  // head 1's keys of the same split, which only query heads 2 and 3 read
  const int nb = (k1 - k0 + 63) / 64;
  const int nbt = two ? 2 * nb : nb;
  for (int j = 0; j < nbt; j += 3) {
    // compute batch j from A while B and C are in flight, then refill A with batch j + 3, and so on
#define MTPD_TEAM_BATCH(J, KR)                                                                                   \
  {                                                                                                              \
    const int g_ = (two && (J) >= nb) ? 1 : 0, t_ = k0 + 64 * ((J) - g_ * nb) + 16 * w;                          \
    if (t_ < k1)                                                                                                 \
      mfma_batch<4, false>(t_, k1, Kb, Kb, cap, true, a.scale_log2, tile, S.qop, KR, KR, acc, mrun, lrun,       \
                           two ? 2 * g_ : 0, two ? 2 * g_ + 2 : 4);                                            \
  }
    MTPD_TEAM_BATCH(j, kA)
    load_key_batch<NKV>(ksp, j + 3, kA);
    MTPD_TEAM_BATCH(j + 1, kB)
    load_key_batch<NKV>(ksp, j + 4, kB);
    MTPD_TEAM_BATCH(j + 2, kC)
    load_key_batch<NKV>(ksp, j + 5, kC);
#undef MTPD_TEAM_BATCH
  }
  if (l == 1) TEAM_TRACE(step, 50);
  if (type) TEAM_TRACE(step, 30);
  if (l == 1) TEAM_TRACE(step, 51);
  // combine the waves: head h's state in lane h; output rows 0..3 (the hi products of heads 0..3) of the tile in
  // lanes 0..15, rows 8..11 (their lo products) in lanes 32..47: both go to LDS and the combine adds them, which
  // costs less than folding the rows across lanes in registers
  float (*wacc)[HD][8] = reinterpret_cast<float (*)[HD][8]>(S.qs_wacc);
  if (lane < 4) {
    S.wml[w][lane][0] = mrun;
    S.wml[w][lane][1] = lrun;
  }
  if (kq == 0 || kq == 2) {
    const int half = kq >> 1;
#pragma unroll
    for (int t = 0; t < TILES; ++t) *reinterpret_cast<f32x4*>(&wacc[w][16 * t + hq][4 * half]) = acc[t];
  }
  __syncthreads();
  if (l == 1) TEAM_TRACE(step, 52);
  {
    const int d = threadIdx.x;
    f32x4 av[4];
    float2 ml[4][4];
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      av[ww] = *reinterpret_cast<const f32x4*>(&wacc[ww][d][0]) + *reinterpret_cast<const f32x4*>(&wacc[ww][d][4]);
#pragma unroll
      for (int hh = 0; hh < 4; ++hh) ml[ww][hh] = *reinterpret_cast<const float2*>(&S.wml[ww][hh][0]);
    }
    const uint32_t tg = T.tag(step, s_att(l));
    uint64_t* ap = T.X + A_AP + T.m * AP_STRIDE;
#pragma unroll
    for (int hh = 0; hh < 4; ++hh) {
      float M = -INFINITY;
#pragma unroll
      for (int ww = 0; ww < 4; ++ww) M = fmaxf(M, ml[ww][hh].x);
      float Ls = 0.f, A = 0.f;
#pragma unroll
      for (int ww = 0; ww < 4; ++ww) {
        const float mw = ml[ww][hh].x;
        const float f = (mw == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mw - M);
        Ls = fmaf(ml[ww][hh].y, f, Ls);
        A = fmaf(av[ww][hh], f, A);
      }
      putf(ap + hh * 258 + d, tg, A);
      if (d == 0) {
        putf(ap + hh * 258 + 256, tg, M);
        putf(ap + hh * 258 + 257, tg, Ls);
      }
    }
  }
  __syncthreads();  // the combine tiles are free again
  if (type) TEAM_TRACE(step, 31);
}

// ------------------------------------------------------------------------------------------------------------
// Merge of a row's key-range partials: o = sum_s 2^(M_s - M) A_s / sum_s 2^(M_s - M) L_s. Member m: 64 (R = 2) or
// 32 (R = 1) dims of one head; wave w takes a quarter of the splits.

template <int R>
__device__ __forceinline__ void stage_mrg(const TeamArgs& a, Team& T, Smem& S, int step, int l) {
  (void)a;
  constexpr int NS = TM / R, SPW = NS / 4, DPB = TQ / (TM / R);
  const int w = wave_id(), lane = lane_id();
  const int r = (R == 2) ? (T.m >> 4) : 0;
  const int d0 = (R == 2) ? 64 * (T.m & 15) : 32 * T.m;
  const int h = d0 >> 8, dd = (d0 & 255) + min(lane, DPB - 1);
  const int b0 = r * NS;  // the row's first attention member
  int idx[SPW + 2];
#pragma unroll
  for (int q = 0; q < SPW; ++q) idx[q] = A_AP + (b0 + w * SPW + q) * AP_STRIDE + h * 258 + dd;
  const int sl = b0 + min(lane, NS - 1);
  idx[SPW] = A_AP + sl * AP_STRIDE + h * 258 + 256;
  idx[SPW + 1] = A_AP + sl * AP_STRIDE + h * 258 + 257;
  uint32_t raw[SPW + 2];
  wait_words<SPW + 2>(T, idx, T.tag(step, s_att(l)), s_att(l), raw);
  if (l == 1) TEAM_TRACE(step, 34);
  const float Ml = __uint_as_float(raw[SPW]), Ll = __uint_as_float(raw[SPW + 1]);
  const float M = wave_max(lane < NS ? Ml : -INFINITY);
  float A = 0.f, Lw = 0.f;
#pragma unroll
  for (int q = 0; q < SPW; ++q) {
    const int sp = w * SPW + q;
    const float ms = readlane_f(Ml, sp), ls = readlane_f(Ll, sp);
    const float f = (ms == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(ms - M);
    A = fmaf(__uint_as_float(raw[q]), f, A);
    Lw = fmaf(ls, f, Lw);
  }
  S.red[w][lane] = A;
  if (lane == 0) S.mrgl[w] = Lw;
  __syncthreads();
  if (w == 0) {
    // the 2048-value output goes out untagged; once wave 0's stores have reached L2, one tagged flag announces them
    // (the consumers then spin on 8 flags instead of re-reading 2048 tagged words)
    if (lane < DPB) {
      const float As = S.red[0][lane] + S.red[1][lane] + S.red[2][lane] + S.red[3][lane];
      const float Ls = S.mrgl[0] + S.mrgl[1] + S.mrgl[2] + S.mrgl[3];
      reinterpret_cast<float*>(T.X + A_O)[r * TQ + d0 + lane] = Ls > 0.f ? As / Ls : 0.f;
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (lane == 0) put(T.X + A_OFL + T.m, T.tag(step, s_mrg(l)), 1u);
  }
  __syncthreads();
}

// ------------------------------------------------------------------------------------------------------------
// 1024 -> 256 products (o_proj over the merged attention output, [MTP doc] "Tensor schema": attn_output; the
// down projection, ffn_down): member m computes outputs 8m .. 8m + 7, wave w the partial over K quarter w.

// The flag a lane of wave w polls before reading quarter w of the merged attention output (dims 256 w .. 256 w + 255
// of each row): member m wrote dims 64 (m mod 16) .. +63 of row m / 16 (R = 2) or dims 32 m .. +31 (R = 1), so the
// quarter's 8 producers are picked by lane mod 8.
template <int R>
__device__ __forceinline__ int mrg_flag() {
  const int w = wave_id(), j = lane_id() & 7;
  if constexpr (R == 2) return (j < 4) ? 4 * w + j : 16 + 4 * w + (j - 4);
  return 8 * w + j;
}

template <int R, bool FLAGGED, typename After>
__device__ __forceinline__ void stage_k1024(Team& T, Smem& S, const WK& W, int src, int flag, uint32_t tag_in,
                                            int sid_in, int dst, uint32_t tag_out, After after_poll) {
  const int w = wave_id(), lane = lane_id();
  const int n0 = 8 * T.m, k = 256 * w + 4 * lane;
  uint32_t raw[R * 4];
  if constexpr (!FLAGGED) {  // tagged input words, polled until every one carries tag_in
    int idx[R * 4];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int e = 0; e < 4; ++e) idx[r * 4 + e] = src + r * 1024 + k + e;
    wait_words<R * 4>(T, idx, tag_in, sid_in, raw);
  } else {  // untagged fp32 pairs: the flags of this wave's quarter's producers, then the quarter, read once from L2
    int fi[1] = {flag};
    uint32_t fr[1];
    wait_words<1>(T, fi, tag_in, sid_in, fr);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const uint64_t p0 = peek(T.X + src + (r * 1024 + k) / 2), p1 = peek(T.X + src + (r * 1024 + k) / 2 + 1);
      raw[r * 4 + 0] = (uint32_t)p0;
      raw[r * 4 + 1] = (uint32_t)(p0 >> 32);
      raw[r * 4 + 2] = (uint32_t)p1;
      raw[r * 4 + 3] = (uint32_t)(p1 >> 32);
    }
  }
  if (sid_in == s_mrg(1)) TEAM_TRACE((int)(tag_in / NSID - T.E - 1), 35);
  if (sid_in == s_ffn(1)) TEAM_TRACE((int)(tag_in / NSID - T.E - 1), 37);
  after_poll();
  float acc[R * 8];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const float4 u = make_float4(__uint_as_float(raw[r * 4]), __uint_as_float(raw[r * 4 + 1]),
                                 __uint_as_float(raw[r * 4 + 2]), __uint_as_float(raw[r * 4 + 3]));
#pragma unroll
    for (int o = 0; o < 8; ++o) acc[r * 8 + o] = dot4(W.w[o], u);
  }
  const int tstep = (int)(tag_in / NSID - T.E - 1);
  if (sid_in == s_mrg(1)) TEAM_TRACE_DEP(tstep, 53, acc[R * 8 - 1]);
  XR<R * 8, 32>::run(acc, lane);
  if (sid_in == s_mrg(1)) TEAM_TRACE_DEP(tstep, 54, acc[0]);
  constexpr int RL = kRedLanes<R>;
  if (lane % RL == 0) S.red[w][lane / RL] = acc[0];
  __syncthreads();
  if (sid_in == s_mrg(1)) TEAM_TRACE(tstep, 55);
  if (threadIdx.x < R * 8) {
    const int i = threadIdx.x;
    putf(T.X + dst + (i >> 3) * TH + n0 + (i & 7), tag_out, S.red[0][i] + S.red[1][i] + S.red[2][i] + S.red[3][i]);
  }
  __syncthreads();
}

// ------------------------------------------------------------------------------------------------------------
// GeGLU FFN input half ([MTP doc] "Tensor schema": post_attention_norm, ffn_norm, ffn_gate, ffn_up; GeGLU is
// gelu_tanh(gate) * up): first the attention residual x = x + RMSNorm(W_o o; post_attention_norm). Member m: ffn
// indices 32m .. 32m + 31.

template <int R>
__device__ __forceinline__ void stage_ffn(const TeamArgs& a, Team& T, Smem& S, int step, int l, const WF& W,
                                          WK& Wd) {
  const int w = wave_id(), lane = lane_id();
  const int f0 = 32 * T.m + 8 * w;
  if (w < R) {
    float d[4];
    poll_row(T, A_T + w * TH, T.tag(step, s_op(l)), s_op(l), d);
    if (l == 1) TEAM_TRACE(step, 36);
    row_update(S, w, 2, d, W.pan, 1.0f, W.fn, a.eps);
    if (l == 1) TEAM_TRACE_DEP(step, 56, S.us[w][lane]);
  }
  issue_k1024(lw(a, l, W_D), T, Wd);  // the down slice, used next stage
  __syncthreads();
  if (l == 1) TEAM_TRACE(step, 57);
  float ag[R * 8], au[R * 8];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const float4 u = *reinterpret_cast<const float4*>(&S.us[r][4 * lane]);
#pragma unroll
    for (int o = 0; o < 8; ++o) {
      ag[r * 8 + o] = dot4(W.g[o], u);
      au[r * 8 + o] = dot4(W.u[o], u);
    }
  }
  if (l == 1) TEAM_TRACE_DEP(step, 58, ag[R * 8 - 1] + au[R * 8 - 1]);
  XR<R * 8, 32>::run(ag, lane);
  XR<R * 8, 32>::run(au, lane);
  if (l == 1) TEAM_TRACE_DEP(step, 59, ag[0] + au[0]);
  constexpr int RL = kRedLanes<R>;
  if (lane % RL == 0) {
    const int i = lane / RL;
    putf(T.X + A_M + (i >> 3) * TF + f0 + (i & 7), T.tag(step, s_ffn(l)), gelu_tanh(ag[0]) * au[0]);
  }
  fill_part<R>(a, T, step, 2 * l + 1, 2 * a.n_layer);  // behind the publish, as in the q stage
  if (l == 1) TEAM_TRACE(step, 60);
}

// ------------------------------------------------------------------------------------------------------------
// Output norm, post_projection and centroid scores ([MTP doc] "Tensor schema": output_norm, assist_post_proj,
// assist_embed_centroids; [Inventory] "Centroid / ordered embeddings LM head", step 1; [Guide] section 6: the
// returned last hidden state is the post-projected one). Member m: Bb / 32 post outputs and 64 centroids; the
// post outputs go out as bf16 pairs, the next step's hidden input.

template <int R, int NBB>
__device__ __forceinline__ void stage_post(const TeamArgs& a, Team& T, Smem& S, int step) {
  WPost<NBB> W;
  issue_post_cen<NBB>(a, T, W);
  constexpr int Bb = NBB * 256, NPB = Bb / 32, NPW = NPB / 4, NPG = (NPW + 7) / 8;
  const int w = wave_id(), lane = lane_id();
  const int last_l = a.n_layer - 1;
  const int p0 = NPB * T.m + NPW * w;  // this wave's first post output
  const int c0 = 64 * T.m + 16 * w;    // this wave's first centroid
  if (w < R) {
    float d[4];
    poll_row(T, A_D + w * TH, T.tag(step, s_dn(last_l)), s_dn(last_l), d);
    TEAM_TRACE(step, 38);
    row_update(S, w, 1, d, W.pfn, a.scale[last_l], W.on, a.eps);
  }

  // this member's -1e30 stores are complete before it publishes anything the head waits for
  if (a.logits) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  issue_post_proj<NBB>(a, T, W);
  __syncthreads();
  constexpr int RL = kRedLanes<R>;
  const bool lastep = step + 1 == a.n_steps;
  float4 u[R];
#pragma unroll
  for (int r = 0; r < R; ++r) u[r] = *reinterpret_cast<const float4*>(&S.us[r][4 * lane]);
  // the centroid scores first: the head waits for them, while the post_projection rows are still arriving
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    float acc[R * 8];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int o = 0; o < 8; ++o) acc[r * 8 + o] = dot4(W.c[g * 8 + o], u[r]);
    XR<R * 8, 32>::run(acc, lane);
    if (lane % RL == 0) {
      const int i = lane / RL;
      reinterpret_cast<float*>(T.X + A_SC)[(i >> 3) * TC + c0 + 8 * g + (i & 7)] = acc[0];
    }
  }
  // the scores go out untagged; once this wave's stores have reached L2, its flag announces them (the head then
  // spins on 32 flags instead of re-reading 2048 tagged words)
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if (lane == 0) put(T.X + A_SFL + 4 * T.m + w, T.tag(step, S_POST), 1u);
#pragma unroll
  for (int g = 0; g < NPG; ++g) {
    float acc[R * 8];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int o = 0; o < 8; ++o) acc[r * 8 + o] = dot4(W.p[g * 8 + o], u[r]);
    XR<R * 8, 32>::run(acc, lane);
    const float nxt = __shfl_down(acc[0], RL, 64);  // output o + 1 of the same row
    const int i = lane / RL, r = i >> 3, o = i & 7;
    if (lane % RL == 0 && (o & 1) == 0 && 8 * g + o < NPW) {
      const int n = p0 + 8 * g + o;
      const uint32_t pair = f2bf2(acc[0], nxt);
      put(T.X + A_HID + r * 2048 + n / 2, T.tag(step, S_POST), pair);
      if (lastep) *reinterpret_cast<uint32_t*>(a.hidden_out + (size_t)T.row(r) * Bb + n) = pair;
    }
  }
}

// ------------------------------------------------------------------------------------------------------------
// The masked head ([Inventory] "Centroid / ordered embeddings LM head", steps 2-5; [Guide] section 5): every
// member ranks its row's 2048 centroid scores (top 32, descending fp32 score, ties to the lower index) and handles
// slots 2 (m mod 16) and 2 (m mod 16) + 1 (R = 2) or slot m (R = 1): the cluster's 128 ids through the ordering, the
// sparse logits E[id] . h from the cluster-ordered table, the scatter into the row, the slot's best (value, id).
//
// Selection, exact: every key is the composite (order-preserving score bits, complement of the index), so the keys
// are distinct and descending key order is descending score with ties to the lower index. Each wave takes a lower
// bound of the 8th largest of its lanes' maximal high halves (at least 8 of its lanes hold a key at or above it);
// the minimum tau of the 4 waves' values therefore has at least 32 keys at or above it, so the 32 largest keys all
// have high half >= tau. Those candidates (typically a few dozen) are ranked by counting the candidates above each
// (all 256 threads at once when there are at most 64).

__device__ __forceinline__ void select_top32(Smem& S, const uint32_t (&ok)[8], const int (&ci)[8], int step) {
  const int tid = threadIdx.x, lane = lane_id(), w = wave_id();
  uint32_t mx = ok[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) mx = max(mx, ok[i]);
  // the wave's 8th largest lane maximum with its low 12 bits cleared, bit by bit from the top: the largest multiple
  // of 2^12 that at least 8 lane maxima reach (the cleared bits only admit a few more candidates)
  uint32_t tw = 0;
  for (int b = 31; b >= 12; --b) {
    const uint32_t cand = tw | (1u << b);
    if (__popcll(__ballot(mx >= cand)) >= 8) tw = cand;
  }
  if (lane == 0) S.wtot[w] = tw;
  if (tid == 0) S.ncand = 0u;
  if (tid < 64) S.cand[tid] = 0ull;  // below every key: the padding of the 64-entry ranking
  __syncthreads();
  TEAM_TRACE(step, 42);
  const uint32_t tau = min(min(S.wtot[0], S.wtot[1]), min(S.wtot[2], S.wtot[3]));
  // append the candidates (their order does not matter): for each of the lane's 8 keys a ballot, the key's place
  // among the wave's set lanes by a count of the lower ones, and one LDS atomic per wave for the base
  uint64_t bal[8];
  uint32_t tot = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    bal[i] = __ballot(ok[i] >= tau);
    tot += (uint32_t)__popcll(bal[i]);
  }
  uint32_t base = 0;
  if (lane == 0) base = atomicAdd(&S.ncand, tot);
  base = (uint32_t)__builtin_amdgcn_readfirstlane((int)base);
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));  // lanes under this one
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (ok[i] >= tau)
      S.cand[base + (uint32_t)__popcll(bal[i] & below)] = ((uint64_t)ok[i] << 32) |
                                                         (uint64_t)(0xFFFFFFFFu - (uint32_t)ci[i]);
    base += (uint32_t)__popcll(bal[i]);
  }
  __syncthreads();
  const uint32_t nc = S.ncand;
  if (nc <= 64) {
    // up to 64 candidates (zero-padded): wave w ranks candidates 16 w + (lane % 16), each lane group of 16 counting
    // the larger ones among 16 of the 64 (reads issued 8 at a time), the 4 groups' counts summed across lanes
    const int e = 16 * w + (lane & 15), fq = lane >> 4;
    const uint64_t me = S.cand[e];
    uint32_t rank = 0;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint64_t o[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) o[j] = S.cand[16 * fq + 8 * h + j];
#pragma unroll
      for (int j = 0; j < 8; ++j) rank += (o[j] > me) ? 1u : 0u;
    }
    rank += __float_as_uint(xr_partner<16>(__uint_as_float(rank)));
    rank += __float_as_uint(xr_partner<32>(__uint_as_float(rank)));
    if (fq == 0 && (uint32_t)e < nc && rank < (uint32_t)TKS)
      S.sel[rank] = (int)(0xFFFFFFFFu - (uint32_t)(me & 0xFFFFFFFFull));
  } else {
    for (uint32_t e = tid; e < nc; e += 256) {
      const uint64_t me = S.cand[e];
      uint32_t rank = 0;
      for (uint32_t f = 0; f < nc; ++f) rank += (S.cand[f] > me) ? 1u : 0u;
      if (rank < (uint32_t)TKS) S.sel[rank] = (int)(0xFFFFFFFFu - (uint32_t)(me & 0xFFFFFFFFull));
    }
  }
  TEAM_TRACE(step, 43);
  __syncthreads();
}

template <int R>
__device__ __forceinline__ void stage_head(const TeamArgs& a, Team& T, Smem& S, int step, uint32_t (&pf)[2]) {
  constexpr int NSL = R;  // slots per member: 2 (R = 2: 16 members per row) or 1 (32 members)
  constexpr int HCH = 2;          // 128-dim chunks of a 256-wide row
  const int tid = threadIdx.x, w = wave_id(), lane = lane_id();
  const int r = (R == 2) ? (T.m >> 4) : 0;
  const int row = T.row(r);
  const int slot0 = (R == 2) ? 2 * (T.m & 15) : T.m;
  // the row's 2048 scores: wave w, centroids 512 w + 64 q + lane
  uint32_t ok[8];
  int ci[8];
  {
    int idx[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      ci[q] = 512 * w + 64 * q + lane;
      idx[q] = r * TC + ci[q];  // fp32 index into the score region
    }
    uint32_t raw[8];
    {
      // this wave's centroids 512 w .. 512 w + 511 come from members 8 w .. 8 w + 7 (all four waves of each): their
      // flags, then the untagged scores, read once from L2
      int fi[1] = {A_SFL + 4 * (8 * w + ((lane >> 2) & 7)) + (lane & 3)};
      uint32_t fr[1];
      wait_words<1>(T, fi, T.tag(step, S_POST), S_POST, fr);
      uint32_t* sc = reinterpret_cast<uint32_t*>(T.X + A_SC);
#pragma unroll
      for (int q = 0; q < 8; ++q) raw[q] = __hip_atomic_load(sc + idx[q], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) ok[q] = f32_order(__uint_as_float(raw[q]));
  }
  TEAM_TRACE(step, 39);
  select_top32(S, ok, ci, step);
  TEAM_TRACE(step, 40);
  // the slots' clusters: group grp (16 lanes) scores ids grp + 16 u, u < 8
  const int grp = tid >> 4, l16 = tid & 15;
  int idv[NSL][8];
  uint4 raw[NSL][8][HCH];
#pragma unroll
  for (int q = 0; q < NSL; ++q) {
    const int c = S.sel[slot0 + q];
    const int32_t* ord = a.ordering + (size_t)c * TVS;
    const uint16_t* crow = a.head_sorted + (size_t)c * TVS * TH;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int t = grp + 16 * u;
      idv[q][u] = ord[t];
#pragma unroll
      for (int ch = 0; ch < HCH; ++ch)
        raw[q][u][ch] = *reinterpret_cast<const uint4*>(crow + (size_t)t * TH + ch * 128 + l16 * 8);
    }
  }
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  float hf[HCH][8];
#pragma unroll
  for (int ch = 0; ch < HCH; ++ch)
#pragma unroll
    for (int e = 0; e < 8; ++e) hf[ch][e] = S.us[r][ch * 128 + l16 * 8 + e];
  const bool want = step + 1 == a.n_steps;  // per-cluster outputs are those of the last step
  TEAM_TRACE(step, 41);
#pragma unroll
  for (int q = 0; q < NSL; ++q) {
    const int slot = slot0 + q;
    float acc[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc[u] = 0.f;
#pragma unroll
    for (int ch = 0; ch < HCH; ++ch)
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        float ef[8];
        unpack8(raw[q][u][ch], ef);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[u] = fmaf(ef[e], hf[ch][e], acc[u]);
      }
    XR<8, 8>::run(acc, l16);  // lane l16 holds id (l16 >> 1) of the group's 8
    const int u = l16 >> 1;
    int idu = idv[q][0];
#pragma unroll
    for (int u2 = 1; u2 < 8; ++u2) idu = (u == u2) ? idv[q][u2] : idu;
    uint64_t best = 0;
    if ((l16 & 1) == 0) {
      const int t = grp + 16 * u;
      if (want) {
        const size_t o = ((size_t)row * TKS + slot) * TVS + t;
        if (a.ids) a.ids[o] = idu;
        if (a.z) a.z[o] = acc[0];
      }
      if (a.logits) a.logits[((size_t)step * a.B + row) * (size_t)a.V + idu] = acc[0];
      best = vid_key(acc[0], (uint32_t)idu);
    }
    best = wave_max_u64(best);
    if (lane == 0) S.bestw[q][w] = best;
  }
  if (tid == 0 && want && a.sel)
    for (int q = 0; q < NSL; ++q) a.sel[(size_t)row * TKS + slot0 + q] = S.sel[slot0 + q];
  __syncthreads();
  if (tid < NSL * 2) {
    const int q = tid >> 1, half = tid & 1;
    const uint64_t k = u64_max(u64_max(S.bestw[q][0], S.bestw[q][1]), u64_max(S.bestw[q][2], S.bestw[q][3]));
    put(T.X + A_KEY + r * (2 * TKS) + 2 * (slot0 + q) + half, T.tag(step, S_KEY),
        half ? (uint32_t)(k >> 32) : (uint32_t)k);
  }
  // The next step's pre reads the target embedding row of the row's token, the best of the 32 slot tokens. Each of
  // this member's slot tokens is a candidate, so wave q touches every 64-byte segment of slot q's row: the row is in
  // the XCD's L2 when the pre stage gathers it. The two words are kept until the next pre stage's waves 0 and 1 have
  // passed their own wait (which covers these loads), so holding them costs no wait.
  if (step + 1 < a.n_steps && w < NSL) {
    const uint64_t k = u64_max(u64_max(S.bestw[w][0], S.bestw[w][1]), u64_max(S.bestw[w][2], S.bestw[w][3]));
    const int t0 = key_id(k);
    const int t = t0 < 0 ? 0 : (t0 >= a.V ? a.V - 1 : t0);
    const uint32_t* er = reinterpret_cast<const uint32_t*>(a.temb + (size_t)t * a.Bb);
    const int nseg = a.Bb / 32;  // 64-byte segments of the row (at most 128)
    pf[0] = er[16 * min(lane, nseg - 1)];
    pf[1] = er[16 * min(64 + lane, nseg - 1)];
  }
  __syncthreads();
}

// The last step's token of each row: the best of its 32 slot keys (member 0 of the team).
template <int R>
__device__ __forceinline__ void stage_final(const TeamArgs& a, Team& T, int step) {
  if (T.m != 0 || wave_id() != 0) return;
  const int lane = lane_id();
  int idx[R];
#pragma unroll
  for (int r = 0; r < R; ++r) idx[r] = A_KEY + r * (2 * TKS) + lane;
  uint32_t raw[R];
  wait_words<R>(T, idx, T.tag(step, S_KEY), S_KEY, raw);
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint32_t lo = pair_lane<0>(raw[r]), hi = pair_lane<1>(raw[r]);
    const int tk = key_id(wave_max_u64(((uint64_t)hi << 32) | lo));
    if (lane == 0) {
      if (a.next) a.next[T.row(r)] = tk;
      if (a.tokens) a.tokens[(size_t)T.row(r) * a.tok_stride + step] = tk;
    }
  }
}

template <int R, int NBB, int NKV>
__device__ __forceinline__ void run_team(const TeamArgs& a, Team& T, Smem& S) {
  WQ wq;
  WK wo, wd;
  WF wf;
  uint32_t pf[2] = {0u, 0u};
  for (int step = 0; step < a.n_steps; ++step) {
    TEAM_TRACE(step, S_PRE);
    TEAM_TRACE_CYCLES(step, 61);
    stage_pre<R, NBB, NKV>(a, T, S, step, wq, pf);
    for (int l = 0; l < a.n_layer; ++l) {
      const bool last = l + 1 == a.n_layer;
      TEAM_TRACE(step, s_q(l));
      stage_q<R>(a, T, S, step, l, wq);
      TEAM_TRACE(step, s_att(l));
      stage_att<R, NKV>(a, T, S, step, l, wo);
      TEAM_TRACE(step, s_mrg(l));
      stage_mrg<R>(a, T, S, step, l);
      TEAM_TRACE(step, s_op(l));
      stage_k1024<R, true>(T, S, wo, A_O, A_OFL + mrg_flag<R>(), T.tag(step, s_mrg(l)), s_mrg(l), A_T, T.tag(step, s_op(l)),
                     [&] { issue_ffn(a, T, l, wf); });
      TEAM_TRACE(step, s_ffn(l));
      stage_ffn<R>(a, T, S, step, l, wf, wd);
      TEAM_TRACE(step, s_dn(l));
      stage_k1024<R, false>(T, S, wd, A_M, 0, T.tag(step, s_ffn(l)), s_ffn(l), A_D, T.tag(step, s_dn(l)), [&] {
        if (!last) issue_q(a, T, l + 1, wq);
      });
    }
    TEAM_TRACE(step, S_POST);
    stage_post<R, NBB>(a, T, S, step);
    TEAM_TRACE(step, S_KEY);
    stage_head<R>(a, T, S, step, pf);
    TEAM_TRACE(step, 27);
    TEAM_TRACE_CYCLES(step, 62);
  }
  stage_final<R>(a, T, a.n_steps - 1);
}

// At least 96 KB of LDS per block keeps one block per CU, so the 256 blocks cover all 256 CUs.
constexpr int kLdsPad = (96 * 1024 > (int)sizeof(Smem)) ? 96 * 1024 - (int)sizeof(Smem) : 0;

// NKV: kv heads (1 or 2), a compile-time constant so that the one-kv-head instance carries none of the second
// head's selects
template <int NBB, int NKV>
__global__ __launch_bounds__(256, 1) void k_team(TeamArgs a) {
  __shared__ Smem S;
  __shared__ uint8_t pad[kLdsPad > 0 ? kLdsPad : 1];
  if (threadIdx.x == 0) pad[0] = 0;
  // The dispatcher deals the blocks out to the XCDs in turn, starting where the previous launch left off: block b
  // runs on XCD (b + k) mod 8 for some k of the launch. The team is the XCD the block runs on (read from the
  // hardware), so a team's 32 blocks share that XCD's L2 and each XCD always uses the same exchange words; b / 8 is
  // then a distinct member index within every team.
  // touch every 64-byte line of the argument block at once: the compiler fetches the arguments lazily, near each
  // use, and at the start of the kernel those fetches would otherwise miss one after another
  {
    constexpr int kLines = (int)((sizeof(TeamArgs) + 63) / 64);
    const uint32_t* kp = (const uint32_t*)__builtin_amdgcn_kernarg_segment_ptr();
    uint32_t t[kLines];
#pragma unroll
    for (int i = 0; i < kLines; ++i) t[i] = kp[16 * i];
#pragma unroll
    for (int i = 0; i < kLines; ++i) asm volatile("" ::"s"(t[i]));
  }
  const uint32_t xcc = (uint32_t)__builtin_amdgcn_s_getreg((20) | (0 << 6) | ((4 - 1) << 11)) & 15u;  // XCC_ID
  Team T;
  T.t = (int)(xcc & (NT - 1));
  T.m = blockIdx.x >> 3;
  T.status = a.status;
  T.dead = false;
  T.X = a.xch + (size_t)T.t * TEAM_WORDS;
  T.E = __hip_atomic_load(a.epoch + blockIdx.x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const bool placed = xcc < (uint32_t)NT;  // else not the 8-XCD layout this kernel is built for: no team work
  if (!placed && threadIdx.x == 0)
    __hip_atomic_fetch_or(a.status, kTeamMisplaced, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  {  // the score tile's unused q columns (head slots 4 .. 7) stay zero for the whole launch
    uint32_t* q = reinterpret_cast<uint32_t*>(&S.qop[0][0][0][0][0]);
    for (int i = threadIdx.x; i < (int)(sizeof(S.qop) / 4); i += 256) q[i] = 0u;
  }
  if (placed && T.t < a.B) {
    T.R = (T.t + NT < a.B) ? 2 : 1;
    T.row0 = T.t;
    T.row1 = T.t + NT;
    if (T.R == 2)
      run_team<2, NBB, NKV>(a, T, S);
    else
      run_team<1, NBB, NKV>(a, T, S);
  }
  __syncthreads();
  if (threadIdx.x == 0) a.epoch[blockIdx.x] = T.E + (uint32_t)a.n_steps;
}

}  // namespace

size_t team_weights_bytes(int Bb) { return w_total(Bb) * sizeof(uint16_t); }

hipError_t team_pack_weights(hipStream_t s, uint16_t* dst, const TeamLayer* L, int n_layer, const uint16_t* pre,
                             const uint16_t* post, const uint16_t* out_norm, const uint16_t* cen, int Bb) {
  auto cp = [&](size_t off, const uint16_t* src, size_t n) {
    return hipMemcpyAsync(dst + off, src, n * sizeof(uint16_t), hipMemcpyDeviceToDevice, s);
  };
  hipError_t e = hipSuccess;
  for (int l = 0; l < n_layer && e == hipSuccess; ++l) {
    const size_t b = (size_t)l * W_LAYER;
    const TeamLayer& y = L[l];
    const struct {
      size_t off;
      const uint16_t* p;
      size_t n;
    } t[10] = {{W_Q, y.q, (size_t)TQ * TH}, {W_QN, y.q_norm, 256},   {W_O, y.o, (size_t)TH * TQ},
               {W_AN, y.attn_norm, TH},     {W_PAN, y.post_attn_norm, TH}, {W_FN, y.ffn_norm, TH},
               {W_PFN, y.post_ffw_norm, TH}, {W_G, y.gate, (size_t)TF * TH}, {W_U, y.up, (size_t)TF * TH},
               {W_D, y.down, (size_t)TH * TF}};
    for (int i = 0; i < 10 && e == hipSuccess; ++i) e = cp(b + t[i].off, t[i].p, t[i].n);
  }
  if (e == hipSuccess) e = cp(W_PRE, pre, (size_t)TH * 2 * Bb);
  if (e == hipSuccess) e = cp(w_post(Bb), post, (size_t)Bb * TH);
  if (e == hipSuccess) e = cp(w_onorm(Bb), out_norm, TH);
  if (e == hipSuccess) e = cp(w_cen(Bb), cen, (size_t)TC * TH);
  return e;
}

size_t team_arena_bytes() { return (size_t)NT * TEAM_WORDS * 8 + (size_t)kTeamBlocks * 4 + 256; }
size_t team_status_offset() { return (size_t)NT * TEAM_WORDS * 8 + (size_t)kTeamBlocks * 4; }

void team_bind_arena(TeamArgs& a, void* arena) {
  uint8_t* p = static_cast<uint8_t*>(arena);
  a.xch = reinterpret_cast<uint64_t*>(p);
  a.epoch = reinterpret_cast<uint32_t*>(p + (size_t)NT * TEAM_WORDS * 8);
  a.status = reinterpret_cast<uint32_t*>(p + team_status_offset());
}

#ifdef MTPD_TEAM_TRACE
hipError_t team_trace_read(uint64_t* host) {
  return hipMemcpyFromSymbol(host, HIP_SYMBOL(g_team_trace), sizeof(uint64_t) * 256 * 256, 0, hipMemcpyDeviceToHost);
}
#endif

bool team_backbone_ok(int Bb) { return Bb == 1536 || Bb == 2048 || Bb == 2560 || Bb == 3072 || Bb == 4096; }

template <int NKV>
hipError_t launch_team_nkv(hipStream_t s, const TeamArgs& a) {
  switch (a.Bb) {
    case 1536: return go(k_team<6, NKV>, dim3(kTeamBlocks), dim3(256), 0, s, a);
    case 2048: return go(k_team<8, NKV>, dim3(kTeamBlocks), dim3(256), 0, s, a);
    case 2560: return go(k_team<10, NKV>, dim3(kTeamBlocks), dim3(256), 0, s, a);
    case 3072: return go(k_team<12, NKV>, dim3(kTeamBlocks), dim3(256), 0, s, a);
    case 4096: return go(k_team<16, NKV>, dim3(kTeamBlocks), dim3(256), 0, s, a);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_team(hipStream_t s, const TeamArgs& a) {
  if (a.nkv == 1) return launch_team_nkv<1>(s, a);
  if (a.nkv == 2) return launch_team_nkv<2>(s, a);
  return hipErrorInvalidValue;
}

}  // namespace mtpd
