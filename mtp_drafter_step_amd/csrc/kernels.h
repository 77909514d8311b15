// Internal launch interface of the drafter-step kernels (gfx950). Host code in runtime.cpp sequences these on a
// stream; every launcher returns the hipError_t of its launch.
//
// Activations are fp32 throughout; stored tensors (weights, caches, embeddings, target hidden) are bf16.
// Kernels never synchronise with each other inside a launch (every cross-block dependency is a kernel boundary),
// except the persistent drafter kernel at the end of this file.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mtpd {

constexpr int kMaxBatch = 256;  // rows per call (matches MTPD_MAX_BATCH)
constexpr int kMaxSplit = 32;  // key-range splits of one (row, kv head)
constexpr int kRowGroup = 4;   // batch rows handled together by the dense kernels
constexpr int kMaxTopK = 64;   // clusters kept per row
constexpr int kMaxCentroids = 4096;
constexpr int kMaxSampleTiles = 256;  // sampled rows hold at most 256 * 4096 scored tokens
constexpr int kGemmMaxK = 8192;      // reduction length of the streaming matrix-core GEMM

// Per-row key window [start, start + count) of one cache, passed by value; start < cap, count <= cap, and indices
// from cap on wrap to slot index - cap.
struct RowWindows {
  int32_t start[kMaxBatch];
  int32_t count[kMaxBatch];
  int32_t shared;  // 1: every row reads cache row 0
};

// Residual update applied in a dense kernel's prologue before its input norm:
//   x_new = (x_old + RMSNorm(delta; w_delta)) * scale       (delta == nullptr: x_new = x_old)
// where delta is the sum of nd partial vectors delta[p * dstride + b * H + i] (p < nd).
struct Residual {
  const float* x_old;       // [B][H]
  const float* delta;       // [nd][B][H] or nullptr
  const uint16_t* w_delta;  // [H]
  float scale;
  float* x_new;             // [B][H], written by one block per row group (nullptr: not stored)
  int nd;                   // partials in delta (1 .. 16)
  size_t dstride;           // elements between consecutive partials
};

// Fill logits[begin, end) with -1e30 (spread over a kernel's blocks; no-op when logits is null).
struct FillRange {
  float* logits;
  size_t begin, end;
};

// Token input of a step: either ids (tok[b]) or, when use_keys is set, the previous step's per-cluster argmax keys
// (keys[b][k]), whose maximum decides the token; in that case block column 0 also records it to out[b*out_stride]
// and next[b]. tok and keys must both be valid device pointers ([B] and [B][k]) whichever is used: both are read.
struct TokenSource {
  const int32_t* tok;
  const uint64_t* keys;
  int use_keys;
  int k;
  int32_t* out;
  int out_stride;
  int32_t* next;
};

// Attach a pair of timing events to the next kernel launched by this thread through one of the launchers below
// (start recorded when the kernel begins, stop when it ends); the pair is consumed by that launch. Null clears.
void set_next_launch_events(hipEvent_t start, hipEvent_t stop);

// x[b] = W_pre [target_hidden[b] ; escale * target_embd[tok[b]]]
hipError_t launch_pre(hipStream_t s, int B, int Bb, int H, int V, const uint16_t* th, TokenSource ts,
                      const uint16_t* emb, float escale, const uint16_t* w_pre, float* x);

// q[b] = W_q RMSNorm(x_new[b]; w_norm)   (raw q, before q_norm and rotation)
hipError_t launch_qproj(hipStream_t s, int B, int H, int QD, Residual res, const uint16_t* w_norm, float eps,
                        const uint16_t* w_q, float* q);

// Single-query attention with q_norm + rotation in the prologue. nsplit == 1: o[b][h*hd + d] directly (fp32);
// nsplit > 1: unnormalised partials (pacc, pml) for launch_attn_merge.
// Whether launch_attn takes the multi-query kernel (a cache shared by the rows, head_dim 256, V = K): its key
// splits then cover the union of the rows' windows.
// valu: the vector-ALU kernel for every shape (the handle option MTPD_OPT_ATTN_VALU).
bool attn_uses_multi_query(bool valu, bool shared, int hd, bool same_v);

// Multi-query attention of rows sharing one cache (head_dim 256, V = K): same inputs and outputs as launch_attn
// with scale_log2 = scale * log2(e).
hipError_t launch_attn_shared(hipStream_t s, int B, int nh, int nkv, const float* q, const uint16_t* qnorm, float eps,
                              const float* rope, int type, const uint16_t* K, int cap, const RowWindows& win,
                              int nsplit, float scale_log2, float* pacc, float* pml, float* o);

hipError_t launch_attn(hipStream_t s, bool valu, int B, int nh, int nkv, int hd, const float* q, const uint16_t* qnorm,
                       float eps, const float* rope, int type, const uint16_t* K, const uint16_t* V, int cap,
                       const RowWindows& win, int nsplit, float scale, float* pacc, float* pml, float* o);

// o_proj in QD / 256 partial sums: t[c][b][n] = sum over k in [256c, 256c + 256) of W[n][k] o[b][k], where o is
// read directly (nsplit == 1) or merged from the attention's split partials (log-sum-exp over the splits of each
// head). W [N][QD]; t [QD / 256][B][N]. The next kernel adds the partials up (Residual::nd).
hipError_t launch_oproj(hipStream_t s, int B, int N, int QD, int hd, int nh, int nsplit, const float* o,
                        const float* pacc, const float* pml, const uint16_t* W, float* t);

// y[b] = W X[b] for fp32 X rows of width K (down: K = ffn; centroid scores: K = hidden), N outputs.
hipError_t launch_dense(hipStream_t s, int B, int K, int N, const float* X, const uint16_t* w, float* y);

// m[b] = gelu_tanh(W_g u) * (W_u u), u = RMSNorm(x_new; w_norm); also fills a slice of the logits.
hipError_t launch_ffn(hipStream_t s, int B, int H, int F, Residual res, const uint16_t* w_norm, float eps,
                      const uint16_t* w_gate, const uint16_t* w_up, float* m, FillRange fill);

// h = RMSNorm(x_new; w_out) (stored to h_out); hidden_out = bf16(W_post h); scores = centroids h (C may be 0);
// keys_zero[0, B) = 0 when set (the dense head's atomic-max keys).
hipError_t launch_post(hipStream_t s, int B, int H, int Bb, int C, Residual res, const uint16_t* w_out, float eps,
                       const uint16_t* w_post, const uint16_t* w_cen, float* h_out, uint16_t* hidden_out,
                       float* scores, uint64_t* keys_zero);

// Dense tied head: logits[b][v] = E[v] . h[b] for every v < V (when logits is set) and keys[b] = max(keys[b],
// (value, id) key of the row's best token); keys must be zero beforehand. V % 16 == 0, H in {256, 512, 768, 1024}.
hipError_t launch_head_dense(hipStream_t s, int B, int V, int H, const uint16_t* E, const float* h, float* logits,
                             uint64_t* keys);

// keys[0, n) = 0
hipError_t launch_zero_keys(hipStream_t s, uint64_t* keys, int n);

// Temperature sampling of one token per row: p = softmax(row / temperature) over the row's scored tokens, drawn
// by inverse CDF at u[b] in the head table's order (k > 0: the masked head's sparse logits vals [B][k][vsc] with
// their ids and the selected clusters sel [B][k], visited by ascending cluster index; k == 0: dense logits vals
// [B][n]). The row maximum comes from keys [B][nk]. tsum: workspace [B][kMaxSampleTiles]. Phase 0 sums the tiles,
// phase 1 draws: it writes the token and its probability at [b * out_stride] of tok_out / prob_out and the token to
// tok_next[b] (each when set).
hipError_t launch_sample(hipStream_t s, int phase, int B, int n, int vsc, int k, const float* vals,
                         const int32_t* ids, const int32_t* sel, const uint64_t* keys, int nk, float temperature,
                         float* tsum, const float* u, int32_t* tok_out, float* prob_out, int out_stride,
                         int32_t* tok_next);

// Masked head: per (row, selected slot j): top-k of the row's centroid scores (descending, ties to the lower
// index), the cluster's token ids through the ordering, sparse logits token_embd[id] . h (rows read from Es, the
// head table in cluster order), optional scatter into logits, and the slot's best (value, id) key (larger value,
// then lower id).
hipError_t launch_head(hipStream_t s, int B, int C, int k, int vsc, int H, const float* scores,
                       const int32_t* ordering, const uint16_t* Es, const float* h, int32_t* sel, int32_t* ids,
                       float* z, float* logits, size_t V, uint64_t* keys);

// The masked head's scoring grouped by cluster (for batches whose rows select many clusters in common):
// launch_topk_rows writes the selections sel [B][k], launch_group groups them by cluster into work (int32, at most
// 4 (C + B k) + B k: a (cluster, first entry, count) record per tile of up to 64 entries of one cluster, then the
// grouped entries), then launch_head_grouped scores them one tile per block, with the same outputs as launch_head.
hipError_t launch_group(hipStream_t s, int B, int C, int k, const int32_t* sel, int32_t* work);
// sel [B][k] = each row's top k of scores [B][C] in slot order (descending score, ties to the lower index).
hipError_t launch_topk_rows(hipStream_t s, int B, int C, int k, const float* scores, int32_t* sel);
hipError_t launch_head_grouped(hipStream_t s, int B, int C, int k, int vsc, int H, const int32_t* ordering,
                               const uint16_t* Es, const float* h, const int32_t* work, int32_t* ids, float* z,
                               float* logits, size_t V, uint64_t* keys);

// out[r] = E[ordering[r]] for r < V (rows of H bf16): the head table in cluster order.
hipError_t launch_gather_rows(hipStream_t s, const uint16_t* E, const int32_t* ordering, uint16_t* out, int V, int H);

// next[b] = token of the largest key in keys[b][0, k); also out2[b*stride2] when set.
hipError_t launch_final(hipStream_t s, int B, int k, const uint64_t* keys, int32_t* next, int32_t* out2, int stride2);

// logits[0, n) = -1e30
hipError_t launch_fill(hipStream_t s, float* logits, size_t n);

// y[b][n] = centroids[n] . h[b] for the masked head on caller-provided states (K = H, N = C).
hipError_t launch_scores(hipStream_t s, int B, int H, int C, const float* h, const uint16_t* w_cen, float* scores);

// ---- dense stages for large batches (k_gemm.hip)

// K chunks for a streaming GEMM of B rows, N outputs and reduction K (1 when the epilogue needs the whole sum).
int gemm_chunks(int B, int N, int K, bool one_chunk);

// Matrix-core GEMM Y = W X^T, W bf16 [N][K], over nchunks K chunks (K % 256 == 0, N % 16 == 0). kind 0: X fp32
// [B][K] -> fp32 partials Y [nchunks][B][N]; 1: -> bf16 Yb [B][N]; 2: GeGLU gelu_tanh(W X) * (W2 X) -> fp32 Y [B][N];
// 3: X = [th ; escale * emb[tok]] (bf16 tables, K = 2 Bb) -> fp32 partials, each row's token taken from ts (the
// caller's or the previous step's argmax, recorded where ts asks; 1 <= ts->k <= 64) and clamped into [0, V). Kinds 1
// and 2 need nchunks == 1. The blocks also fill a slice of the logits with -1e30 (fill.logits null: none).
hipError_t launch_gemm(hipStream_t s, int kind, int B, int N, int K, const float* X, const uint16_t* th,
                       const uint16_t* emb, const TokenSource* ts, int Bb, float escale, const uint16_t* W,
                       const uint16_t* W2, float* Y, uint16_t* Yb, int nchunks, FillRange fill = FillRange{nullptr, 0, 0},
                       int V = 0);

// Per row: x = sum of nx partials of xp (stride xs); with delta (nd partials, stride ds) x = (x + RMSNorm(delta;
// w_delta)) * scale; x_new = x (when set); u = RMSNorm(x; w_norm); keys_zero[b] = 0 (when set). H % 256 == 0.
hipError_t launch_rownorm(hipStream_t s, int B, int H, const float* xp, int nx, size_t xs, const float* delta, int nd,
                          size_t ds, const uint16_t* w_delta, float scale, const uint16_t* w_norm, float eps,
                          float* x_new, float* u, uint64_t* keys_zero);

// o[b][h] = merge of the nsplit key-range partials (pacc, pml) of the attention.
hipError_t launch_merge(hipStream_t s, int B, int nh, int hd, int nsplit, const float* pacc, const float* pml, float* o);

// ---- persistent drafter kernel (k_team.hip)
//
// One launch runs n whole drafter steps for up to kTeamMaxBatch rows. The grid is one block per CU of the 8 XCDs
// (256 blocks of 256 threads); the 32 blocks of XCD t form team t and compute rows t and t + 8. Inside a team,
// every value one block hands to another is a 64-bit word (fp32 or packed bits, 32-bit tag) stored into the XCD's
// L2 and polled with device-coherent loads; tags are unique per (launch, step, stage), so the exchange buffers never
// need clearing. Every wait is bounded: a wait that runs out sets `status` and the launch finishes with undefined
// outputs instead of hanging.

constexpr int kTeamMaxBatch = 16;
constexpr int kTeamMaxLayers = 4;
constexpr int kTeamBlocks = 256;
// status bits
constexpr uint32_t kTeamTimeout = 1u;    // a wait ran out (the first stage id that did is in status[1] + 1)
constexpr uint32_t kTeamMisplaced = 2u;  // a block ran on an XCD outside the 8 the teams are built for

struct TeamLayer {
  const uint16_t *q, *q_norm, *o, *attn_norm, *post_attn_norm, *ffn_norm, *post_ffw_norm, *gate, *up, *down;
  float scale;
};

struct TeamArgs {
  const uint16_t* wpk;  // the dense weights packed by team_pack_weights (one base pointer: compile-time offsets)
  float scale[kTeamMaxLayers];  // layer_output_scale
  const uint16_t* head_sorted;
  const int32_t* ordering;
  const uint16_t* th;    // [B][Bb] step-0 hidden input
  const int32_t* tok;    // [B] step-0 token
  const uint16_t* temb;  // [V][Bb]
  const uint16_t* kc[2];  // per-row caches [B][nkv][cap][256], K = V (0 sliding, 1 full)
  int32_t cap[2];
  int32_t win_start[2][kTeamMaxBatch], win_count[2][kTeamMaxBatch];
  const float* rope;  // [B][2][2][128]
  float* logits;      // [n][B][V] or null
  int32_t* tokens;    // tokens[b * tok_stride + i] = step i's token (null: not stored)
  int32_t tok_stride;
  int32_t* next;          // [B] the last step's token (null: not stored)
  uint16_t* hidden_out;   // [B][Bb] of the last step
  int32_t* sel;           // [B][32] (null: not stored)
  int32_t* ids;           // [B][32][128] (null: not stored)
  float* z;               // [B][32][128] (null: not stored)
  int32_t B, n_steps, n_layer, Bb, V;
  int32_t nkv;  // kv heads: 1 (4 query heads per kv head) or 2 (query heads 2 g, 2 g + 1 read kv head g)
  uint32_t full_mask;
  float eps, scale_log2, escale;
  uint64_t* xch;     // exchange words, team_arena_words() per team
  uint32_t* epoch;   // [kTeamBlocks] per-block launch counters (zero at creation)
  uint32_t* status;  // [2]
};

// The persistent kernel reads the dense weights (every layer's q / norms / o / gate / up / down, pre_proj,
// post_proj, output_norm, centroids) from one buffer of team_weights_bytes(Bb); team_pack_weights fills it with
// device-to-device copies on stream s.
size_t team_weights_bytes(int Bb);
hipError_t team_pack_weights(hipStream_t s, uint16_t* dst, const TeamLayer* L, int n_layer, const uint16_t* pre,
                             const uint16_t* post, const uint16_t* out_norm, const uint16_t* cen, int Bb);
// Bytes of the arena (exchange words, epochs, status) the persistent kernel needs; must be zeroed once before the
// first launch and then only used by this kernel.
size_t team_arena_bytes();
// Point a's exchange words, epochs and status into an arena of team_arena_bytes(); the status words sit at byte
// team_status_offset() of it.
void team_bind_arena(TeamArgs& a, void* arena);
size_t team_status_offset();
// Whether a backbone width has a persistent-kernel instance.
bool team_backbone_ok(int Bb);
hipError_t launch_team(hipStream_t s, const TeamArgs& a);
#ifdef MTPD_TEAM_TRACE
hipError_t team_trace_read(uint64_t* host);  // measurement builds: the last launch's stage timeline
#endif

// Measurement helper (k_stream.hip): read `bytes` (a multiple of 16, 16-byte aligned buffer) with streaming vector
// loads; sink[0] is written only if the xor of all words equals key.
hipError_t launch_stream_read(hipStream_t s, const void* buf, uint64_t bytes, uint32_t key, uint32_t* sink);

}  // namespace mtpd
