// Host runtime of the drafter-step library: argument validation, workspace plan and kernel sequencing behind the
// C ABI declared in include/mtpd.h.
//
// Pages cited (by title; sections as headed on each page):
//   [MTP doc]    "Gemma 4 Multi-Token Prediction (MTP) drafter" (llama.cpp fork, gemma4-assistant.md)
//   [Inventory]  "Gemma 4 Assistant (MTP drafter) - tensor inventory (Stage 0)"
//   [Guide]      "Gemma 4 Assistant 使用指南：用 MTP 投机解码与 KV Sharing 加速 Gemma 4 推理" (gitcode blog)
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "kernels.h"
#include "mtpd.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

// Scratch memory of the allocation-free entry point (mtpd_drafter_step_noalloc): a file-scope device array, one copy
// per device, held until the process ends. In host code the name `scratch` is a host-side stand-in, never a device
// address: host code uses only the per-device address resolved by scratch_setup().
constexpr size_t kScratchBytes = MTPD_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

// While set on this thread, the call in progress launches its kernels directly on the caller's stream (no graph is
// captured or instantiated, both of which allocate) and takes no timing records (their events are created lazily).
thread_local bool t_direct = false;

constexpr int kGraphCache = 32;
constexpr int kChains = 4;  // maximum sub-batches (make_chains currently uses one: graph replays on separate streams
                            // were measured not to overlap)

// Everything a captured call depends on: the graph of one (call, arguments) pair is replayed only when every
// pointer, size and per-row window is the same.
struct CallKey {
  int32_t kind, batch, n, chain;
  const void* ptrs[16];
  mtpd::RowWindows win[2];
  int32_t nsplit[2];
  int32_t caps[2];
  uint32_t fbits;  // bits of a float argument baked into the kernels (the sampling temperature), else 0
  bool operator==(const CallKey& o) const { return std::memcmp(this, &o, sizeof(CallKey)) == 0; }
};

struct GraphEntry {
  CallKey key;
  hipGraphExec_t exec = nullptr;
  uint64_t used = 0;
};

}  // namespace

struct mtpd_handle_s {
  mtpd_config cfg;
  mtpd_weights w;
  std::vector<mtpd_layer> layers;
  int32_t max_batch;
  int32_t vsc;
  uint16_t* head_sorted = nullptr;  // token_embd rows in cluster order (owned; built by mtpd_create)
  bool use_graphs = true;
  // the persistent drafter kernel (k_team.hip): whether the configuration has an instance, whether it is enabled,
  // and its arena (exchange words, per-block epochs, status), zeroed at creation
  bool team_shape = false;
  bool team_enabled = true;  // MTPD_OPT_PERSISTENT
  int dense_path = 0;        // MTPD_OPT_DENSE_PATH: 0 by batch size, 1 fused small-batch kernels, 2 matrix-core GEMMs
  bool attn_valu = false;    // MTPD_OPT_ATTN_VALU
  uint8_t* team_arena = nullptr;
  uint16_t* team_weights = nullptr;  // the dense weights packed in the persistent kernel's layout (owned)
  hipStream_t cap_stream = nullptr;
  GraphEntry graphs[kGraphCache];
  uint64_t tick = 0;
  // independent row chains run on their own streams, forked from and joined back into the caller's stream
  hipStream_t chain_stream[kChains] = {};
  hipEvent_t fork_ev = nullptr;
  hipEvent_t join_ev[kChains] = {};
  // kernel timing: while `timing` is set every launch takes the next event pair and records its site label
  mutable bool timing = false;
  mutable int32_t n_timed = 0;
  mutable std::vector<hipEvent_t> timing_ev;  // 2 per record, created on first use
  mutable std::vector<const char*> timing_name;
};

namespace {

size_t align_up(size_t x) { return (x + 255) & ~size_t(255); }

// Offsets of every intermediate in the caller's workspace for a given batch.
struct Plan {
  size_t x[2], q, pacc, pml, o, t, m, d, h, hid, tok, scores, sel, ids, z, keys, stok, tsum, row, u, xp, dp,
      grp, total;
};

// Argmax keys per row: one per selected cluster for the masked head, one for the dense head.
int key_slots(const mtpd_config& c) { return c.n_centroids == 0 ? 1 : c.top_k; }

Plan make_plan(const mtpd_config& c, int B, int vsc) {
  Plan p{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += align_up(bytes);
    return o;
  };
  const size_t H = c.hidden, Bb = c.backbone, QD = (size_t)c.n_head * c.head_dim, F = c.ffn;
  p.x[0] = take((size_t)B * H * 4);
  p.x[1] = take((size_t)B * H * 4);
  p.q = take((size_t)B * QD * 4);
  p.pacc = take((size_t)B * c.n_head * mtpd::kMaxSplit * c.head_dim * 4);
  p.pml = take((size_t)B * c.n_head * mtpd::kMaxSplit * 2 * 4);
  p.o = take((size_t)B * QD * 4);
  p.t = take((size_t)(QD / 256) * B * H * 4);  // o_proj partials [QD / 256][B][H]
  p.m = take((size_t)B * F * 4);
  p.d = take((size_t)B * H * 4);
  p.h = take((size_t)B * H * 4);
  p.hid = take((size_t)2 * B * Bb * 2);
  p.tok = take((size_t)2 * B * 4);
  p.scores = take((size_t)B * c.n_centroids * 4);
  p.sel = take((size_t)B * c.top_k * 4);
  p.ids = take((size_t)B * c.top_k * vsc * 4);
  p.z = take((size_t)B * c.top_k * vsc * 4);
  p.keys = take((size_t)B * key_slots(c) * 8);
  p.stok = take((size_t)B * 4);                                  // sampled tokens (next step's input)
  p.tsum = take((size_t)B * mtpd::kMaxSampleTiles * 4);          // sampling tile sums
  p.row = take(c.n_centroids == 0 ? (size_t)B * c.vocab * 4 : 0);  // dense logits rows for sampling
  // the large-batch path: normed stage inputs, K-split partials of pre_projection and down, resolved tokens
  p.u = take((size_t)B * H * 4);
  p.xp = take((size_t)(2 * Bb / 256) * B * H * 4);
  p.dp = take((size_t)(F / 256) * B * H * 4);
  // cluster grouping of the head: a 16-byte record per (cluster, entry tile), then the grouped entries
  p.grp = take((size_t)(4 * (c.n_centroids + B * std::max(c.top_k, 1)) + B * std::max(c.top_k, 1)) * 4);
  p.total = off;
  return p;
}

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

int check_config(const mtpd_config* c) {
  if (!c) return fail(MTPD_EINVAL, "config is NULL");
  const bool dense = c->n_centroids == 0;  // dense tied head
  if (c->backbone <= 0 || c->hidden <= 0 || c->n_layer <= 0 || c->n_head <= 0 || c->n_kv_head <= 0 ||
      c->head_dim <= 0 || c->ffn <= 0 || c->vocab <= 0 || c->n_centroids < 0 || c->swa_window <= 0 ||
      (!dense && c->top_k <= 0))
    return fail(MTPD_ESHAPE, "every size in the config must be positive (n_centroids may be 0: dense head)");
  if (dense) {
    if (c->top_k != 0 && c->top_k != 1) return fail(MTPD_ESHAPE, "top_k must be 0 or 1 with the dense head");
    if (c->vocab % 16 != 0) return fail(MTPD_ESHAPE, "vocab must be a multiple of 16 with the dense head");
  } else {
    if (c->vocab % c->n_centroids != 0) return fail(MTPD_ESHAPE, "vocab %% n_centroids != 0");
    if (c->top_k > c->n_centroids) return fail(MTPD_ESHAPE, "top_k > n_centroids");
  }
  if (c->n_head % c->n_kv_head != 0) return fail(MTPD_ESHAPE, "n_head %% n_kv_head != 0");
  const int G = c->n_head / c->n_kv_head;
  if (G != 1 && G != 2 && G != 4 && G != 8) return fail(MTPD_ESHAPE, "query heads per kv head must be 1, 2, 4 or 8");
  if (c->head_dim != 64 && c->head_dim != 128 && c->head_dim != 256)
    return fail(MTPD_ESHAPE, "head_dim must be 64, 128 or 256");
  if (c->hidden % 256 != 0 || c->hidden > 1024) return fail(MTPD_ESHAPE, "hidden must be a multiple of 256, <= 1024");
  if (c->backbone % 256 != 0 || c->backbone > 8192)
    return fail(MTPD_ESHAPE, "backbone must be a multiple of 256, <= 8192");
  if (c->ffn % 256 != 0 || c->ffn > 4096) return fail(MTPD_ESHAPE, "ffn must be a multiple of 256, <= 4096");
  if ((c->n_head * c->head_dim) % 256 != 0 || c->n_head * c->head_dim > 4096)
    return fail(MTPD_ESHAPE, "n_head*head_dim must be a multiple of 256, <= 4096");
  if (!dense) {
    if (c->n_centroids > mtpd::kMaxCentroids) return fail(MTPD_ESHAPE, "n_centroids > 4096");
    if (c->top_k > mtpd::kMaxTopK) return fail(MTPD_ESHAPE, "top_k > 64");
    const int vsc = c->vocab / c->n_centroids;
    if (vsc % 16 != 0 || vsc > 1024)
      return fail(MTPD_ESHAPE, "vocab / n_centroids must be a multiple of 16, <= 1024");
  }
  if (c->n_layer > 32) return fail(MTPD_ESHAPE, "n_layer > 32");
  if (!(c->rms_eps >= 0.f) || !(c->attn_scale > 0.f)) return fail(MTPD_EINVAL, "rms_eps < 0 or attn_scale <= 0");
  return MTPD_OK;
}

int check_ptr(const void* p, const char* name) {
  if (!p) return fail(MTPD_EINVAL, "%s is NULL", name);
  if (!aligned16(p)) return fail(MTPD_EINVAL, "%s is not 16-byte aligned", name);
  return MTPD_OK;
}

#define CHECK(expr)                 \
  do {                              \
    int rc_ = (expr);               \
    if (rc_ != MTPD_OK) return rc_; \
  } while (0)

#define LAUNCH(expr)                                                                        \
  do {                                                                                      \
    hipError_t e_ = (expr);                                                                 \
    if (e_ != hipSuccess) return fail(MTPD_EHIP, "%s: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

// Take the next timing record for a launch labelled `name` (no-op unless timing is on; launches beyond
// MTPD_MAX_TIMED records are not recorded).
int timing_mark(const mtpd_handle_s* h, const char* name) {
  if (t_direct || !h->timing || h->n_timed >= MTPD_MAX_TIMED) return MTPD_OK;
  const size_t i = (size_t)h->n_timed;
  if (h->timing_ev.size() < 2 * (i + 1)) {
    for (int j = 0; j < 2; ++j) {
      hipEvent_t e = nullptr;
      LAUNCH(hipEventCreate(&e));
      h->timing_ev.push_back(e);
    }
    h->timing_name.push_back(nullptr);
  }
  h->timing_name[i] = name;
  mtpd::set_next_launch_events(h->timing_ev[2 * i], h->timing_ev[2 * i + 1]);
  ++h->n_timed;
  return MTPD_OK;
}

// A kernel launch labelled for the timing records.
#define KLAUNCH(h, name, expr)                                                                \
  do {                                                                                        \
    CHECK(timing_mark((h), (name)));                                                          \
    hipError_t e_ = (expr);                                                                   \
    mtpd::set_next_launch_events(nullptr, nullptr);                                           \
    if (e_ != hipSuccess) return fail(MTPD_EHIP, "%s: %s", #expr, hipGetErrorString(e_));   \
  } while (0)

int check_kv(const mtpd_handle_s* h, const mtpd_kv& kv, int B, const char* name, mtpd::RowWindows* win, bool full) {
  char nm[64];
  snprintf(nm, sizeof(nm), "%s.k", name);
  CHECK(check_ptr(kv.k, nm));
  snprintf(nm, sizeof(nm), "%s.v", name);
  CHECK(check_ptr(kv.v, nm));
  if (!kv.len) return fail(MTPD_EINVAL, "%s.len is NULL", name);
  if (kv.cap <= 0) return fail(MTPD_ESHAPE, "%s.cap must be positive", name);
  std::memset(win, 0, sizeof(*win));
  win->shared = kv.shared ? 1 : 0;
  for (int b = 0; b < B; ++b) {
    const int L = kv.len[b];
    if (L < 1 || L > kv.cap) return fail(MTPD_ESHAPE, "%s.len[%d] = %d outside [1, cap=%d]", name, b, L, kv.cap);
    const int f = kv.first ? kv.first[b] : 0;
    if (f < 0 || f >= kv.cap) return fail(MTPD_ESHAPE, "%s.first[%d] = %d outside [0, cap=%d)", name, b, f, kv.cap);
    // the last n valid keys; window indices from cap on wrap to the start of the cache
    const int n = full ? L : std::min(L, h->cfg.swa_window);
    const int s0 = f + (L - n);
    win->start[b] = s0 >= kv.cap ? s0 - kv.cap : s0;
    win->count[b] = n;
  }
  return MTPD_OK;
}

// Splits of each row's key window. A block of the attention kernel runs 4 waves that take 16-key batches in turn,
// and each batch costs about one memory round trip, so a block should see few batches; but every block pays the
// same prologue, and the split partials are merged by a second kernel. Blocks cover at least 64 keys (one batch
// per wave) and at least the batch's keys / 256 (about one block per CU), up to kMaxSplit blocks per
// (row, kv head).
int nsplit_for(const mtpd::RowWindows& win, int B, int nkv) {
  int mx = 1;
  long total = 0;
  for (int b = 0; b < B; ++b) {
    mx = std::max(mx, win.count[b]);
    total += win.count[b];
  }
  const long per = std::max<long>(64, (total * nkv + 255) / 256);
  const long ns = (mx + per - 1) / per;
  return (int)std::max<long>(1, std::min<long>(ns, mtpd::kMaxSplit));
}

// The masked head on fp32 hidden states h [B][H] and centroid scores already in the workspace: per (row, slot)
// top-k + gather + dot (+ scatter) and the slot's best (value, id) key. With few rows one kernel does it all per
// (row, slot); with many (B k at least the cluster count) the selection runs once per row, the selections are
// grouped by cluster, and each cluster's rows are read once for all the rows that chose it.
int run_head(const mtpd_handle_s* h, hipStream_t s, void* ws, const Plan& p, int B, const float* hsrc,
             float* logits, int32_t* sel_out, int32_t* ids_out, float* z_out) {
  const mtpd_config& c = h->cfg;
  if (c.n_centroids == 0) {  // dense tied head ([Guide] section 5, use_ordered_embeddings off); keys zeroed before
    KLAUNCH(h, "head_dense", mtpd::launch_head_dense(s, B, c.vocab, c.hidden, h->w.token_embd, hsrc, logits,
                                                     at<uint64_t>(ws, p.keys)));
    return MTPD_OK;
  }
  // [Inventory] "Centroid / ordered embeddings LM head", steps 2-5
  if (B * c.top_k >= c.n_centroids) {  // many rows: the selected clusters read once, scored for every row
    int32_t* selw = sel_out ? sel_out : at<int32_t>(ws, p.sel);
    KLAUNCH(h, "head_select", mtpd::launch_topk_rows(s, B, c.n_centroids, c.top_k, at<float>(ws, p.scores), selw));
    KLAUNCH(h, "head_group", mtpd::launch_group(s, B, c.n_centroids, c.top_k, selw, at<int32_t>(ws, p.grp)));
    KLAUNCH(h, "head_grouped", mtpd::launch_head_grouped(s, B, c.n_centroids, c.top_k, h->vsc, c.hidden,
                                                         h->w.token_ordering, h->head_sorted, hsrc,
                                                         at<int32_t>(ws, p.grp), ids_out, z_out, logits,
                                                         (size_t)c.vocab, at<uint64_t>(ws, p.keys)));
    return MTPD_OK;
  }
  KLAUNCH(h, "head", mtpd::launch_head(s, B, c.n_centroids, c.top_k, h->vsc, c.hidden, at<float>(ws, p.scores),
                           h->w.token_ordering, h->head_sorted, hsrc, sel_out, ids_out, z_out, logits,
                           (size_t)c.vocab, at<uint64_t>(ws, p.keys)));
  return MTPD_OK;
}

// One drafter step on workspace buffers: input hidden `th` [B][Bb], token source `ts`; leaves the per-slot argmax
// keys in the workspace (the step's token is their maximum). Small batches: kernels that fold each stage's residual
// and norm into their prologue.
int run_step_small(const mtpd_handle_s* h, hipStream_t s, void* ws, const Plan& p, int B, const uint16_t* th,
             mtpd::TokenSource ts, const uint16_t* temb, const mtpd_shared_kv* kv, const mtpd::RowWindows* win,
             const int* nsplit, float* logits, uint16_t* hidden_out, int32_t* sel_out, int32_t* ids_out,
             float* z_out) {
  const mtpd_config& c = h->cfg;
  const int H = c.hidden, Bb = c.backbone, QD = c.n_head * c.head_dim, F = c.ffn, nL = c.n_layer;
  float* x[2] = {at<float>(ws, p.x[0]), at<float>(ws, p.x[1])};
  float* q = at<float>(ws, p.q);
  float* o = at<float>(ws, p.o);
  float* t = at<float>(ws, p.t);
  float* m = at<float>(ws, p.m);
  float* d = at<float>(ws, p.d);
  // input assembly + pre_projection ([MTP doc] "What it is"; [Guide] section 2(3))
  KLAUNCH(h, "pre", mtpd::launch_pre(s, B, Bb, H, c.vocab, th, ts, temb, c.embed_scale, h->w.pre_proj, x[0]));
  int cur = 0;
  const size_t BV = (size_t)B * c.vocab;
  for (int l = 0; l < nL; ++l) {
    const mtpd_layer& L = h->layers[l];
    const int type = ((c.full_attn_layers >> l) & 1u) ? 1 : 0;
    const mtpd_kv& cache = type ? kv->full : kv->sliding;
    mtpd::Residual rq{x[cur], nullptr, nullptr, 1.0f, nullptr, 1, 0};
    if (l > 0) {
      const mtpd_layer& P = h->layers[l - 1];
      rq = mtpd::Residual{x[cur], d, P.post_ffw_norm, P.layer_output_scale, x[cur ^ 1], 1, 0};
      cur ^= 1;
    }
    KLAUNCH(h, "qproj", mtpd::launch_qproj(s, B, H, QD, rq, L.attn_norm, c.rms_eps, L.attn_q, q));
    KLAUNCH(h, type ? "attn_full" : "attn_sliding", mtpd::launch_attn(s, h->attn_valu, B, c.n_head, c.n_kv_head, c.head_dim, q, L.attn_q_norm, c.rms_eps, kv->rope, type,
                             cache.k, cache.v, cache.cap, win[type], nsplit[type], c.attn_scale,
                             at<float>(ws, p.pacc), at<float>(ws, p.pml), o));
    // o_proj in QD / 256 partials, merging the split attention partials on the way in
    KLAUNCH(h, "o_proj", mtpd::launch_oproj(s, B, H, QD, c.head_dim, c.n_head, nsplit[type], o, at<float>(ws, p.pacc),
                                            at<float>(ws, p.pml), L.attn_output, t));
    mtpd::Residual rf{x[cur], t, L.post_attention_norm, 1.0f, x[cur ^ 1], QD / 256, (size_t)B * H};
    cur ^= 1;
    mtpd::FillRange fr{nullptr, 0, 0};
    if (logits && c.n_centroids > 0)  // the dense head writes every logit itself
      fr = mtpd::FillRange{logits, (BV * l / nL) & ~size_t(3), l + 1 == nL ? BV : (BV * (l + 1) / nL) & ~size_t(3)};
    KLAUNCH(h, "ffn", mtpd::launch_ffn(s, B, H, F, rf, L.ffn_norm, c.rms_eps, L.ffn_gate, L.ffn_up, m, fr));
    KLAUNCH(h, "down", mtpd::launch_dense(s, B, F, H, m, L.ffn_down, d));
  }
  const mtpd_layer& Last = h->layers[nL - 1];
  mtpd::Residual rp{x[cur], d, Last.post_ffw_norm, Last.layer_output_scale, nullptr, 1, 0};
  // output norm, post_projection (the next step's hidden input, [Guide] section 6) and centroid scores
  KLAUNCH(h, "post", mtpd::launch_post(s, B, H, Bb, c.n_centroids, rp, h->w.output_norm, c.rms_eps, h->w.post_proj,
                           h->w.centroids, at<float>(ws, p.h), hidden_out, at<float>(ws, p.scores),
                           c.n_centroids == 0 ? at<uint64_t>(ws, p.keys) : nullptr));
  return run_head(h, s, ws, p, B, at<float>(ws, p.h), logits, sel_out, ids_out, z_out);
}

// Batches of at least this many rows take the matrix-core path for the dense stages (the handle option
// MTPD_OPT_DENSE_PATH forces either path).
constexpr int kGemmRows = 32;

bool use_gemm_path(const mtpd_handle_s* h, int B) {
  // the pre_projection GEMM takes K = 2 * backbone <= 8192; wider backbones keep the small-batch kernels
  if (2 * h->cfg.backbone > mtpd::kGemmMaxK) return false;
  if (h->dense_path == 1) return false;
  if (h->dense_path == 2) return true;
  return B >= kGemmRows;
}

// One drafter step with the dense stages as streaming matrix-core GEMMs (large batches): a residual + norm kernel
// per stage feeds each GEMM its normed input once; K-split partials are summed by the next norm kernel.
int run_step_gemm(const mtpd_handle_s* h, hipStream_t s, void* ws, const Plan& p, int B, const uint16_t* th,
                  mtpd::TokenSource ts, const uint16_t* temb, const mtpd_shared_kv* kv, const mtpd::RowWindows* win,
                  const int* nsplit, float* logits, uint16_t* hidden_out, int32_t* sel_out, int32_t* ids_out,
                  float* z_out) {
  const mtpd_config& c = h->cfg;
  const int H = c.hidden, Bb = c.backbone, QD = c.n_head * c.head_dim, F = c.ffn, nL = c.n_layer;
  const bool dense = c.n_centroids == 0;
  const size_t BH = (size_t)B * H;
  float* x = at<float>(ws, p.x[0]);
  float* u = at<float>(ws, p.u);
  float* q = at<float>(ws, p.q);
  float* o = at<float>(ws, p.o);
  float* t = at<float>(ws, p.t);
  float* m = at<float>(ws, p.m);
  float* xp = at<float>(ws, p.xp);
  float* dp = at<float>(ws, p.dp);
  // input assembly + pre_projection ([MTP doc] "What it is"; [Guide] section 2(3)); the GEMM's blocks resolve the
  // rows' tokens themselves
  const int npre = mtpd::gemm_chunks(B, H, 2 * Bb, false);
  KLAUNCH(h, "pre_gemm", mtpd::launch_gemm(s, 3, B, H, 2 * Bb, nullptr, th, temb, &ts, Bb, c.embed_scale, h->w.pre_proj,
                                           nullptr, xp, nullptr, npre, mtpd::FillRange{nullptr, 0, 0}, c.vocab));
  const float* xin = xp;  // the residual stream entering the next norm, as partials
  int nx = npre;
  const float* din = nullptr;
  int nd = 1;
  const uint16_t* wd = nullptr;
  float sc = 1.0f;
  const int no = mtpd::gemm_chunks(B, H, QD, false), nf = mtpd::gemm_chunks(B, H, F, false);
  // the masked head's -1e30 base row, written in 4 nL slices by the blocks of the layers' four GEMMs (the dense head
  // writes every logit itself)
  const size_t BV = (size_t)B * c.vocab;
  const int nslice = 4 * nL;
  auto fill_slice = [&](int i) {
    if (!logits || dense) return mtpd::FillRange{nullptr, 0, 0};
    const size_t a = (BV * (size_t)i / nslice) & ~size_t(3);
    const size_t e = i + 1 == nslice ? BV : (BV * (size_t)(i + 1) / nslice) & ~size_t(3);
    return mtpd::FillRange{logits, a, e};
  };
  for (int l = 0; l < nL; ++l) {
    const mtpd_layer& L = h->layers[l];
    const int type = ((c.full_attn_layers >> l) & 1u) ? 1 : 0;
    const mtpd_kv& cache = type ? kv->full : kv->sliding;
    KLAUNCH(h, "rownorm", mtpd::launch_rownorm(s, B, H, xin, nx, BH, din, nd, BH, wd, sc, L.attn_norm, c.rms_eps, x, u,
                                               nullptr));
    KLAUNCH(h, "qproj_gemm", mtpd::launch_gemm(s, 0, B, QD, H, u, nullptr, nullptr, nullptr, 0, 0.f, L.attn_q, nullptr,
                                               q, nullptr, 1, fill_slice(4 * l)));
    KLAUNCH(h, type ? "attn_full" : "attn_sliding",
            mtpd::launch_attn(s, h->attn_valu, B, c.n_head, c.n_kv_head, c.head_dim, q, L.attn_q_norm, c.rms_eps, kv->rope, type,
                              cache.k, cache.v, cache.cap, win[type], nsplit[type], c.attn_scale, at<float>(ws, p.pacc),
                              at<float>(ws, p.pml), o));
    if (nsplit[type] > 1)
      KLAUNCH(h, "attn_merge", mtpd::launch_merge(s, B, c.n_head, c.head_dim, nsplit[type], at<float>(ws, p.pacc),
                                                  at<float>(ws, p.pml), o));
    KLAUNCH(h, "o_proj_gemm", mtpd::launch_gemm(s, 0, B, H, QD, o, nullptr, nullptr, nullptr, 0, 0.f, L.attn_output,
                                                nullptr, t, nullptr, no, fill_slice(4 * l + 1)));
    KLAUNCH(h, "rownorm", mtpd::launch_rownorm(s, B, H, x, 1, 0, t, no, BH, L.post_attention_norm, 1.0f, L.ffn_norm,
                                               c.rms_eps, x, u, nullptr));
    KLAUNCH(h, "ffn_gemm", mtpd::launch_gemm(s, 2, B, F, H, u, nullptr, nullptr, nullptr, 0, 0.f, L.ffn_gate, L.ffn_up,
                                             m, nullptr, 1, fill_slice(4 * l + 2)));
    KLAUNCH(h, "down_gemm", mtpd::launch_gemm(s, 0, B, H, F, m, nullptr, nullptr, nullptr, 0, 0.f, L.ffn_down, nullptr,
                                              dp, nullptr, nf, fill_slice(4 * l + 3)));
    xin = x;
    nx = 1;
    din = dp;
    nd = nf;
    wd = L.post_ffw_norm;
    sc = L.layer_output_scale;
  }
  // output norm, post_projection (the next step's hidden input, [Guide] section 6) and centroid scores
  KLAUNCH(h, "post_norm", mtpd::launch_rownorm(s, B, H, xin, nx, BH, din, nd, BH, wd, sc, h->w.output_norm, c.rms_eps,
                                               nullptr, at<float>(ws, p.h), dense ? at<uint64_t>(ws, p.keys) : nullptr));
  KLAUNCH(h, "post_gemm", mtpd::launch_gemm(s, 1, B, Bb, H, at<float>(ws, p.h), nullptr, nullptr, nullptr, 0, 0.f,
                                            h->w.post_proj, nullptr, nullptr, hidden_out, 1));
  if (!dense && c.n_centroids % 16 != 0) {
    KLAUNCH(h, "scores", mtpd::launch_scores(s, B, H, c.n_centroids, at<float>(ws, p.h), h->w.centroids,
                                             at<float>(ws, p.scores)));
  } else if (!dense) {
    KLAUNCH(h, "scores_gemm", mtpd::launch_gemm(s, 0, B, c.n_centroids, H, at<float>(ws, p.h), nullptr, nullptr, nullptr,
                                                0, 0.f, h->w.centroids, nullptr, at<float>(ws, p.scores), nullptr, 1));
  }
  return run_head(h, s, ws, p, B, at<float>(ws, p.h), logits, sel_out, ids_out, z_out);
}

int run_step(const mtpd_handle_s* h, hipStream_t s, void* ws, const Plan& p, int B, const uint16_t* th,
             mtpd::TokenSource ts, const uint16_t* temb, const mtpd_shared_kv* kv, const mtpd::RowWindows* win,
             const int* nsplit, float* logits, uint16_t* hidden_out, int32_t* sel_out, int32_t* ids_out,
             float* z_out) {
  if (use_gemm_path(h, B))
    return run_step_gemm(h, s, ws, p, B, th, ts, temb, kv, win, nsplit, logits, hidden_out, sel_out, ids_out, z_out);
  return run_step_small(h, s, ws, p, B, th, ts, temb, kv, win, nsplit, logits, hidden_out, sel_out, ids_out, z_out);
}

int check_call(const mtpd_handle_s* h, void* ws, int B) {
  if (!h) return fail(MTPD_EINVAL, "handle is NULL");
  if (B < 1 || B > h->max_batch) return fail(MTPD_ESHAPE, "batch %d outside [1, max_batch=%d]", B, h->max_batch);
  if (!ws) return fail(MTPD_EINVAL, "workspace is NULL");
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0) return fail(MTPD_EINVAL, "workspace is not 256-byte aligned");
  return MTPD_OK;
}

// The per-cluster outputs exist only for the masked head.
int check_head_outputs(const mtpd_handle_s* h, const void* sel, const void* ids, const void* z) {
  if (h->cfg.n_centroids == 0 && (sel || ids || z))
    return fail(MTPD_EINVAL, "sel_centroids / sparse_ids / sparse_logits must be NULL with the dense head");
  return MTPD_OK;
}

// Splits of the union of the rows' windows for the multi-query attention (rows sharing one cache): about 256 blocks
// over the (split, 128-query group, kv head) grid, at least 64 keys per split.
int nsplit_multi_query(const mtpd::RowWindows& win, int B, int G, int nkv) {
  int u0 = win.start[0], u1 = win.start[0] + win.count[0];
  for (int b = 1; b < B; ++b) {
    u0 = std::min(u0, win.start[b]);
    u1 = std::max(u1, win.start[b] + win.count[b]);
  }
  const int groups = (B + 8 * (16 / G) - 1) / (8 * (16 / G)) * nkv;
  const int ns = std::max(1, std::min((256 + groups - 1) / groups, (u1 - u0 + 63) / 64));
  return std::min(ns, mtpd::kMaxSplit);
}

int split_count(const mtpd_handle_s* h, const mtpd_kv& kv, const mtpd::RowWindows& win, int B) {
  const mtpd_config& c = h->cfg;
  if (mtpd::attn_uses_multi_query(h->attn_valu, kv.shared != 0, c.head_dim, kv.v == kv.k))
    return nsplit_multi_query(win, B, c.n_head / c.n_kv_head, c.n_kv_head);
  return nsplit_for(win, B, c.n_kv_head);
}

int check_step_inputs(const mtpd_handle_s* h, int B, const uint16_t* th, const int32_t* tok, const uint16_t* temb,
                      const mtpd_shared_kv* kv, mtpd::RowWindows* win, int* nsplit) {
  CHECK(check_ptr(th, "target_hidden"));
  if (!tok) return fail(MTPD_EINVAL, "last_token is NULL");
  CHECK(check_ptr(temb, "target_embd"));
  if (!kv) return fail(MTPD_EINVAL, "shared kv is NULL");
  if (!kv->rope) return fail(MTPD_EINVAL, "rope is NULL");
  CHECK(check_kv(h, kv->sliding, B, "sliding", &win[0], false));
  CHECK(check_kv(h, kv->full, B, "full", &win[1], true));
  nsplit[0] = split_count(h, kv->sliding, win[0], B);
  nsplit[1] = split_count(h, kv->full, win[1], B);
  return MTPD_OK;
}

// Rows are independent, so a batch is cut into up to kChains sub-batches (multiples of the 4-row group) whose
// kernel chains run concurrently: every stage is latency-bound, and one chain's memory waits overlap the others'
// work. Each chain has its own workspace region.
struct Chains {
  int n;
  int rows[kChains + 1];
  int bmax;
};

Chains make_chains(int B) {
  Chains c{};
  const int per = B;  // one chain: see kChains
  c.n = (B + per - 1) / per;
  for (int i = 0; i <= c.n; ++i) c.rows[i] = std::min(B, i * per);
  c.bmax = std::min(per, B);
  return c;
}

// The rows [b0, b0 + Bc) of the shared caches, rotary tables and key windows.
struct ChainView {
  mtpd_shared_kv kv;
  mtpd::RowWindows win[2];
  int nsplit[2];
};

ChainView chain_view(const mtpd_handle_s* h, const mtpd_shared_kv* kv, const mtpd::RowWindows* win, int b0, int Bc) {
  ChainView v;
  v.kv = *kv;
  const size_t hd = (size_t)h->cfg.head_dim, nkv = (size_t)h->cfg.n_kv_head;
  const size_t ss = nkv * (size_t)kv->sliding.cap * hd, fs = nkv * (size_t)kv->full.cap * hd;
  const size_t bs = kv->sliding.shared ? 0 : b0, bf = kv->full.shared ? 0 : b0;  // shared caches: one row
  v.kv.sliding.k = kv->sliding.k + bs * ss;
  v.kv.sliding.v = kv->sliding.v + bs * ss;
  v.kv.full.k = kv->full.k + bf * fs;
  v.kv.full.v = kv->full.v + bf * fs;
  v.kv.sliding.len = kv->sliding.len + b0;
  v.kv.full.len = kv->full.len + b0;
  if (kv->sliding.first) v.kv.sliding.first = kv->sliding.first + b0;
  if (kv->full.first) v.kv.full.first = kv->full.first + b0;
  v.kv.rope = kv->rope + (size_t)b0 * 2 * hd;
  for (int t = 0; t < 2; ++t) {
    std::memset(&v.win[t], 0, sizeof(v.win[t]));
    v.win[t].shared = win[t].shared;
    for (int i = 0; i < Bc; ++i) {
      v.win[t].start[i] = win[t].start[b0 + i];
      v.win[t].count[i] = win[t].count[b0 + i];
    }
    v.nsplit[t] = split_count(h, t ? kv->full : kv->sliding, v.win[t], Bc);
  }
  return v;
}

// body(chain, stream) for every chain: forked from `s` by an event, joined back by events.
template <typename Body>
int run_chains(mtpd_handle_s* h, hipStream_t s, const Chains& ch, Body body) {
  if (ch.n == 1) return body(0, s);
  if (!h->fork_ev) {
    LAUNCH(hipEventCreateWithFlags(&h->fork_ev, hipEventDisableTiming));
    for (int c = 0; c < kChains; ++c) {
      LAUNCH(hipStreamCreateWithFlags(&h->chain_stream[c], hipStreamNonBlocking));
      LAUNCH(hipEventCreateWithFlags(&h->join_ev[c], hipEventDisableTiming));
    }
  }
  LAUNCH(hipEventRecord(h->fork_ev, s));
  for (int c = 0; c < ch.n; ++c) {
    LAUNCH(hipStreamWaitEvent(h->chain_stream[c], h->fork_ev, 0));
    CHECK(body(c, h->chain_stream[c]));
    LAUNCH(hipEventRecord(h->join_ev[c], h->chain_stream[c]));
  }
  for (int c = 0; c < ch.n; ++c) LAUNCH(hipStreamWaitEvent(s, h->join_ev[c], 0));
  return MTPD_OK;
}

// Find or capture the graph of one chain of a call.
template <typename Body>
int chain_graph(mtpd_handle_s* h, const CallKey& key, int chain, Body body, hipGraphExec_t* out) {
  CallKey k = key;
  k.chain = chain;
  for (auto& e : h->graphs)
    if (e.exec && e.key == k) {
      e.used = ++h->tick;
      *out = e.exec;
      return MTPD_OK;
    }
  if (!h->cap_stream) LAUNCH(hipStreamCreateWithFlags(&h->cap_stream, hipStreamNonBlocking));
  GraphEntry* slot = &h->graphs[0];
  for (auto& e : h->graphs) {
    if (!e.exec) {
      slot = &e;
      break;
    }
    if (e.used < slot->used) slot = &e;
  }
  LAUNCH(hipStreamBeginCapture(h->cap_stream, hipStreamCaptureModeThreadLocal));
  int rc = body(chain, h->cap_stream);
  hipGraph_t graph = nullptr;
  hipError_t e = hipStreamEndCapture(h->cap_stream, &graph);
  if (rc != MTPD_OK) {
    if (graph) (void)hipGraphDestroy(graph);
    return rc;
  }
  if (e != hipSuccess) return fail(MTPD_EHIP, "hipStreamEndCapture: %s", hipGetErrorString(e));
  hipGraphExec_t exec = nullptr;
  e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
  (void)hipGraphDestroy(graph);
  if (e != hipSuccess) return fail(MTPD_EHIP, "hipGraphInstantiate: %s", hipGetErrorString(e));
  if (slot->exec) (void)hipGraphExecDestroy(slot->exec);
  slot->key = k;
  slot->exec = exec;
  slot->used = ++h->tick;
  *out = exec;
  return MTPD_OK;
}

// Run a call made of independent row chains, body(chain, stream) launching one chain's kernels, on the caller's
// stream `s`. Each chain is replayed from its own captured graph (captured on first use) on its own stream, forked
// from and joined back into `s` by events, so that the chains' kernels overlap. When the caller's stream is being
// captured, or graphs are off, the chains' kernels are launched directly on the forked streams.
template <typename Body>
int run_call(mtpd_handle_s* h, hipStream_t s, const CallKey& key, const Chains& ch, Body body) {
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &st) != hipSuccess) st = hipStreamCaptureStatusActive;
  if (t_direct || !h->use_graphs || h->timing || st != hipStreamCaptureStatusNone) return run_chains(h, s, ch, body);
  hipGraphExec_t exec[kChains];
  for (int c = 0; c < ch.n; ++c) CHECK(chain_graph(h, key, c, body, &exec[c]));
  if (ch.n == 1) {
    LAUNCH(hipGraphLaunch(exec[0], s));
    return MTPD_OK;
  }
  return run_chains(h, s, ch, [&](int c, hipStream_t cs) -> int {
    LAUNCH(hipGraphLaunch(exec[c], cs));
    return MTPD_OK;
  });
}

// Bytes reserved for the persistent kernel's arena (at the start of the allocation-free entry point's scratch and of
// each handle's own arena allocation).
size_t team_arena_span() { return align_up(mtpd::team_arena_bytes()); }

// Resolve the current device's copy of `scratch` (once per device; called by mtpd_create with the device current).
int scratch_setup() {
  int dev = -1;
  LAUNCH(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return fail(MTPD_EUNSUP, "device %d: at most %d devices are supported", dev, kMaxDevices);
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if (g_scratch_dev[dev]) return MTPD_OK;
  void* ptr = nullptr;
  hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess || !ptr) return fail(MTPD_EHIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
  // the persistent kernel's arena at the start of the array must start out zero (epochs, tags, status)
  e = hipMemset(ptr, 0, team_arena_span());
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) return fail(MTPD_EHIP, "clearing the scratch arena: %s", hipGetErrorString(e));
  g_scratch_dev[dev] = ptr;
  return MTPD_OK;
}

// The current device's scratch address, or nullptr if no handle was created on this device.
void* scratch_lookup() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> g(g_scratch_mu);
  return g_scratch_dev[dev];
}

// The persistent kernel's shapes: the E2B / E4B drafters (hidden 256, 4 heads of 256 over one or two K = V heads,
// FFN 1024, 2048 clusters of 128 tokens, top 32, at most 4 layers) on a gfx950 with 256 CUs (8 XCDs of 32).
bool team_config_ok(const mtpd_config& c) {
  return c.hidden == 256 && c.n_head == 4 && (c.n_kv_head == 1 || c.n_kv_head == 2) && c.head_dim == 256 &&
         c.ffn == 1024 &&
         c.n_layer >= 1 && c.n_layer <= mtpd::kTeamMaxLayers && c.n_centroids == 2048 && c.top_k == 32 &&
         c.vocab == 2048 * 128 && mtpd::team_backbone_ok(c.backbone);
}

bool team_device_ok() {
  int dev = -1;
  hipDeviceProp_t p;
  if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&p, dev) != hipSuccess) return false;
  return p.multiProcessorCount == mtpd::kTeamBlocks && std::strncmp(p.gcnArchName, "gfx950", 6) == 0;
}

// The arena the persistent kernel uses on this call: the allocation-free entry point's, else the handle's.
thread_local uint8_t* t_arena = nullptr;

bool team_call_ok(const mtpd_handle_s* h, int B, const mtpd_shared_kv* kv) {
  return h->team_shape && h->team_enabled && B <= mtpd::kTeamMaxBatch && !kv->sliding.shared && !kv->full.shared &&
         kv->sliding.v == kv->sliding.k && kv->full.v == kv->full.k;
}

// n drafter steps of B rows in one launch of the persistent kernel. Step i's token goes to tokens[b * n + i] and the
// last step's to next[b] (each when set); logits [n][B][V]; sel / ids / z of the last step.
int run_team(const mtpd_handle_s* h, hipStream_t s, int B, int n, const uint16_t* th, const int32_t* tok,
             const uint16_t* temb, const mtpd_shared_kv* kv, const mtpd::RowWindows* win, float* logits,
             int32_t* tokens, int32_t* next, uint16_t* hidden_out, int32_t* sel, int32_t* ids, float* z) {
  const mtpd_config& c = h->cfg;
  mtpd::TeamArgs a;
  std::memset(&a, 0, sizeof(a));
  for (int l = 0; l < c.n_layer; ++l) a.scale[l] = h->layers[l].layer_output_scale;
  a.wpk = h->team_weights;
  a.head_sorted = h->head_sorted;
  a.ordering = h->w.token_ordering;
  a.th = th;
  a.tok = tok;
  a.temb = temb;
  a.kc[0] = kv->sliding.k;
  a.kc[1] = kv->full.k;
  a.cap[0] = kv->sliding.cap;
  a.cap[1] = kv->full.cap;
  for (int t = 0; t < 2; ++t)
    for (int b = 0; b < B; ++b) {
      a.win_start[t][b] = win[t].start[b];
      a.win_count[t][b] = win[t].count[b];
    }
  a.rope = kv->rope;
  a.logits = logits;
  a.tokens = tokens;
  a.tok_stride = n;
  a.next = next;
  a.hidden_out = hidden_out;
  a.sel = sel;
  a.ids = ids;
  a.z = z;
  a.B = B;
  a.n_steps = n;
  a.n_layer = c.n_layer;
  a.Bb = c.backbone;
  a.V = c.vocab;
  a.nkv = c.n_kv_head;
  a.full_mask = c.full_attn_layers;
  a.eps = c.rms_eps;
  a.scale_log2 = c.attn_scale * 1.4426950408889634f;
  a.escale = c.embed_scale;
  mtpd::team_bind_arena(a, t_arena ? t_arena : h->team_arena);
  KLAUNCH(h, "team", mtpd::launch_team(s, a));
  return MTPD_OK;
}

CallKey make_key(int kind, int B, int n, std::initializer_list<const void*> ptrs, const mtpd::RowWindows* win,
                 const int* nsplit, const mtpd_shared_kv* kv, float farg = 0.f) {
  CallKey k;
  std::memset(&k, 0, sizeof(k));
  std::memcpy(&k.fbits, &farg, sizeof(farg));
  k.kind = kind;
  k.chain = -1;
  k.batch = B;
  k.n = n;
  int i = 0;
  for (const void* p : ptrs) k.ptrs[i++] = p;
  if (win) {
    k.win[0] = win[0];
    k.win[1] = win[1];
    k.nsplit[0] = nsplit[0];
    k.nsplit[1] = nsplit[1];
  }
  if (kv) {
    k.caps[0] = kv->sliding.cap;
    k.caps[1] = kv->full.cap;
  }
  return k;
}

}  // namespace

extern "C" {

int32_t mtpd_abi_version(void) { return 6; }

const char* mtpd_last_error(void) { return g_last_error.c_str(); }

int mtpd_create(const mtpd_config* cfg, const mtpd_weights* w, int32_t max_batch, mtpd_handle* out) {
  g_last_error.clear();
  if (!out) return fail(MTPD_EINVAL, "out is NULL");
  *out = nullptr;
  CHECK(check_config(cfg));
  if (!w) return fail(MTPD_EINVAL, "weights are NULL");
  if (max_batch < 1 || max_batch > MTPD_MAX_BATCH) return fail(MTPD_ESHAPE, "max_batch outside [1, %d]", MTPD_MAX_BATCH);
  CHECK(check_ptr(w->pre_proj, "pre_proj"));
  CHECK(check_ptr(w->post_proj, "post_proj"));
  CHECK(check_ptr(w->output_norm, "output_norm"));
  CHECK(check_ptr(w->token_embd, "token_embd"));
  const bool dense = cfg->n_centroids == 0;  // centroids and token_ordering are not read by the dense head
  if (!dense) {
    CHECK(check_ptr(w->centroids, "centroids"));
    CHECK(check_ptr(w->token_ordering, "token_ordering"));
  }
  if (!w->layers) return fail(MTPD_EINVAL, "layers is NULL");
  for (int l = 0; l < cfg->n_layer; ++l) {
    const mtpd_layer& L = w->layers[l];
    const void* ps[10] = {L.attn_q, L.attn_q_norm, L.attn_output, L.attn_norm, L.post_attention_norm,
                          L.ffn_norm, L.post_ffw_norm, L.ffn_gate, L.ffn_up, L.ffn_down};
    static const char* names[10] = {"attn_q", "attn_q_norm", "attn_output", "attn_norm", "post_attention_norm",
                                    "ffn_norm", "post_ffw_norm", "ffn_gate", "ffn_up", "ffn_down"};
    for (int i = 0; i < 10; ++i) {
      char nm[64];
      snprintf(nm, sizeof(nm), "layers[%d].%s", l, names[i]);
      CHECK(check_ptr(ps[i], nm));
    }
  }
  CHECK(scratch_setup());  // the allocation-free entry point's scratch on this device (after all host-side checks)
  if (!dense) {
    // token_ordering must list every token once ([Inventory] "GGUF / converter layout", verification)
    std::vector<int32_t> ord((size_t)cfg->vocab);
    hipError_t e = hipMemcpy(ord.data(), w->token_ordering, ord.size() * sizeof(int32_t), hipMemcpyDeviceToHost);
    if (e != hipSuccess) return fail(MTPD_EHIP, "copying token_ordering: %s", hipGetErrorString(e));
    std::vector<uint8_t> seen((size_t)cfg->vocab, 0);
    for (size_t i = 0; i < ord.size(); ++i) {
      const int32_t v = ord[i];
      if (v < 0 || v >= cfg->vocab || seen[(size_t)v])
        return fail(MTPD_ESHAPE, "token_ordering is not a permutation (entry %zu = %d)", i, v);
      seen[(size_t)v] = 1;
    }
  }
  mtpd_handle_s* hh = new (std::nothrow) mtpd_handle_s();
  if (!hh) return fail(MTPD_ENOMEM, "out of host memory");
  if (!dense) {
    // the head table in cluster order ([Inventory] "Centroid / ordered embeddings LM head", step 3: a cluster's
    // ids are a contiguous slice of the ordering), so that a selected cluster's rows are one contiguous read
    const size_t head_bytes = (size_t)cfg->vocab * cfg->hidden * sizeof(uint16_t);
    if (hipMalloc(&hh->head_sorted, head_bytes) != hipSuccess) {
      delete hh;
      return fail(MTPD_ENOMEM, "no device memory for the cluster-ordered head table (%zu bytes)", head_bytes);
    }
    hipError_t e =
        mtpd::launch_gather_rows(nullptr, w->token_embd, w->token_ordering, hh->head_sorted, cfg->vocab, cfg->hidden);
    if (e == hipSuccess) e = hipStreamSynchronize(nullptr);
    if (e != hipSuccess) {
      (void)hipFree(hh->head_sorted);
      delete hh;
      return fail(MTPD_EHIP, "building the cluster-ordered head table: %s", hipGetErrorString(e));
    }
  }
  hh->cfg = *cfg;
  hh->w = *w;
  hh->layers.assign(w->layers, w->layers + cfg->n_layer);
  hh->w.layers = nullptr;
  hh->max_batch = max_batch;
  hh->vsc = dense ? 0 : cfg->vocab / cfg->n_centroids;
  hh->team_shape = team_config_ok(*cfg) && team_device_ok();
  if (hh->team_shape) {
    if (hipMalloc(&hh->team_arena, team_arena_span()) != hipSuccess) {
      mtpd_destroy(hh);
      return fail(MTPD_ENOMEM, "no device memory for the persistent kernel's arena (%zu bytes)", team_arena_span());
    }
    if (hipMalloc(&hh->team_weights, mtpd::team_weights_bytes(cfg->backbone)) != hipSuccess) {
      mtpd_destroy(hh);
      return fail(MTPD_ENOMEM, "no device memory for the persistent kernel's packed weights (%zu bytes)",
                  mtpd::team_weights_bytes(cfg->backbone));
    }
    mtpd::TeamLayer tl[mtpd::kTeamMaxLayers];
    for (int l = 0; l < cfg->n_layer; ++l) {
      const mtpd_layer& L = hh->layers[l];
      tl[l] = mtpd::TeamLayer{L.attn_q, L.attn_q_norm, L.attn_output, L.attn_norm, L.post_attention_norm,
                              L.ffn_norm, L.post_ffw_norm, L.ffn_gate, L.ffn_up, L.ffn_down, L.layer_output_scale};
    }
    hipError_t e = mtpd::team_pack_weights(nullptr, hh->team_weights, tl, cfg->n_layer, w->pre_proj, w->post_proj,
                                           w->output_norm, w->centroids, cfg->backbone);
    if (e == hipSuccess) e = hipMemset(hh->team_arena, 0, team_arena_span());
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) {
      mtpd_destroy(hh);
      return fail(MTPD_EHIP, "clearing the persistent kernel's arena: %s", hipGetErrorString(e));
    }
  }
  *out = hh;
  return MTPD_OK;
}

void mtpd_destroy(mtpd_handle h) {
  if (!h) return;
  for (auto& e : h->graphs)
    if (e.exec) (void)hipGraphExecDestroy(e.exec);
  if (h->cap_stream) (void)hipStreamDestroy(h->cap_stream);
  for (int c = 0; c < kChains; ++c) {
    if (h->chain_stream[c]) (void)hipStreamDestroy(h->chain_stream[c]);
    if (h->join_ev[c]) (void)hipEventDestroy(h->join_ev[c]);
  }
  if (h->fork_ev) (void)hipEventDestroy(h->fork_ev);
  for (hipEvent_t e : h->timing_ev) (void)hipEventDestroy(e);
  if (h->head_sorted) (void)hipFree(h->head_sorted);
  if (h->team_arena) (void)hipFree(h->team_arena);
  if (h->team_weights) (void)hipFree(h->team_weights);
  delete h;
}

size_t mtpd_workspace_bytes(mtpd_handle h, int32_t batch) {
  if (!h || batch < 1 || batch > h->max_batch) return 0;
  const Chains ch = make_chains(batch);
  return (size_t)ch.n * make_plan(h->cfg, ch.bmax, h->vsc).total;
}

int mtpd_drafter_step(mtpd_handle h, void* stream, void* workspace, int32_t batch, const uint16_t* target_hidden,
                      const int32_t* last_token, const uint16_t* target_embd, const mtpd_shared_kv* kv,
                      float* logits, int32_t* next_token, uint16_t* hidden_out, int32_t* sel_centroids,
                      int32_t* sparse_ids, float* sparse_logits) {
  g_last_error.clear();
  CHECK(check_call(h, workspace, batch));
  mtpd::RowWindows win[2];
  int nsplit[2];
  CHECK(check_step_inputs(h, batch, target_hidden, last_token, target_embd, kv, win, nsplit));
  if (!next_token) return fail(MTPD_EINVAL, "next_token is NULL");
  CHECK(check_ptr(hidden_out, "hidden_out"));
  if (logits) CHECK(check_ptr(logits, "logits"));
  CHECK(check_head_outputs(h, sel_centroids, sparse_ids, sparse_logits));
  if (team_call_ok(h, batch, kv))
    return run_team(h, static_cast<hipStream_t>(stream), batch, 1, target_hidden, last_token, target_embd, kv, win,
                    logits, nullptr, next_token, hidden_out, sel_centroids, sparse_ids, sparse_logits);
  const Chains ch = make_chains(batch);
  const Plan p = make_plan(h->cfg, ch.bmax, h->vsc);
  const CallKey key = make_key(1, batch, 1,
                               {workspace, target_hidden, last_token, target_embd, kv->sliding.k, kv->sliding.v,
                                kv->full.k, kv->full.v, kv->rope, logits, next_token, hidden_out, sel_centroids,
                                sparse_ids, sparse_logits},
                               win, nsplit, kv);
  const mtpd_config& c = h->cfg;
  const size_t kv_n = (size_t)c.top_k * h->vsc;
  return run_call(h, static_cast<hipStream_t>(stream), key, ch, [&](int ci, hipStream_t cs) -> int {
      const int b0 = ch.rows[ci], Bc = ch.rows[ci + 1] - b0;
      void* wsc = static_cast<char*>(workspace) + (size_t)ci * p.total;
      const ChainView v = chain_view(h, kv, win, b0, Bc);
      mtpd::TokenSource ts{last_token + b0, at<uint64_t>(wsc, p.keys), 0, key_slots(c), nullptr, 0, nullptr};
      CHECK(run_step(h, cs, wsc, p, Bc, target_hidden + (size_t)b0 * c.backbone, ts, target_embd, &v.kv, v.win,
                     v.nsplit, logits ? logits + (size_t)b0 * c.vocab : nullptr,
                     hidden_out + (size_t)b0 * c.backbone, sel_centroids ? sel_centroids + (size_t)b0 * c.top_k : nullptr,
                     sparse_ids ? sparse_ids + b0 * kv_n : nullptr, sparse_logits ? sparse_logits + b0 * kv_n : nullptr));
      KLAUNCH(h, "final", mtpd::launch_final(cs, Bc, key_slots(c), at<uint64_t>(wsc, p.keys), next_token + b0, nullptr, 0));
      return MTPD_OK;
  });
}

int mtpd_drafter_step_noalloc(mtpd_handle h, void* stream, int32_t batch, const uint16_t* target_hidden,
                              const int32_t* last_token, const uint16_t* target_embd, const mtpd_shared_kv* kv,
                              float* logits, int32_t* next_token, uint16_t* hidden_out, int32_t* sel_centroids,
                              int32_t* sparse_ids, float* sparse_logits) {
  g_last_error.clear();
  if (!h) return fail(MTPD_EINVAL, "handle is NULL");
  uint8_t* sc = static_cast<uint8_t*>(scratch_lookup());
  if (!sc) return fail(MTPD_EINVAL, "no handle was created on the current device, so its scratch is not set up");
  // the persistent kernel's arena first, then the workspace of the other paths
  void* ws = sc + team_arena_span();
  const size_t room = kScratchBytes - team_arena_span();
  const size_t need = mtpd_workspace_bytes(h, batch);
  if (need == 0) return fail(MTPD_ESHAPE, "batch %d outside [1, max_batch=%d]", batch, h->max_batch);
  if (need > room)
    return fail(MTPD_ESHAPE, "batch %d needs %zu bytes of scratch; the allocation-free entry point holds %zu", batch,
                need, room);
  struct Direct {
    uint8_t* saved;
    explicit Direct(uint8_t* arena) : saved(t_arena) {
      t_direct = true;
      t_arena = arena;
    }
    ~Direct() {
      t_direct = false;
      t_arena = saved;
    }
  } direct(sc);
  return mtpd_drafter_step(h, stream, ws, batch, target_hidden, last_token, target_embd, kv, logits, next_token,
                           hidden_out, sel_centroids, sparse_ids, sparse_logits);
}

int mtpd_draft_block(mtpd_handle h, void* stream, void* workspace, int32_t batch, int32_t n,
                     const uint16_t* target_hidden, const int32_t* last_token, const uint16_t* target_embd,
                     const mtpd_shared_kv* kv, int32_t* tokens, float* logits, uint16_t* hidden_out) {
  g_last_error.clear();
  CHECK(check_call(h, workspace, batch));
  if (n < 1 || n > 64) return fail(MTPD_ESHAPE, "n must be in [1, 64]");
  mtpd::RowWindows win[2];
  int nsplit[2];
  CHECK(check_step_inputs(h, batch, target_hidden, last_token, target_embd, kv, win, nsplit));
  if (!tokens) return fail(MTPD_EINVAL, "tokens is NULL");
  CHECK(check_ptr(hidden_out, "hidden_out"));
  if (logits) CHECK(check_ptr(logits, "logits"));
  if (team_call_ok(h, batch, kv))
    return run_team(h, static_cast<hipStream_t>(stream), batch, n, target_hidden, last_token, target_embd, kv, win,
                    logits, tokens, nullptr, hidden_out, nullptr, nullptr, nullptr);
  const Chains ch = make_chains(batch);
  const Plan p = make_plan(h->cfg, ch.bmax, h->vsc);
  const mtpd_config& c = h->cfg;
  const size_t BV = (size_t)batch * c.vocab;
  const CallKey key = make_key(2, batch, n,
                               {workspace, target_hidden, last_token, target_embd, kv->sliding.k, kv->sliding.v,
                                kv->full.k, kv->full.v, kv->rope, logits, tokens, hidden_out},
                               win, nsplit, kv);
  return run_call(h, static_cast<hipStream_t>(stream), key, ch, [&](int ci, hipStream_t cs) -> int {
      const int b0 = ch.rows[ci], Bc = ch.rows[ci + 1] - b0;
      void* wsc = static_cast<char*>(workspace) + (size_t)ci * p.total;
      const ChainView v = chain_view(h, kv, win, b0, Bc);
      uint16_t* hid[2] = {at<uint16_t>(wsc, p.hid), at<uint16_t>(wsc, p.hid) + (size_t)Bc * c.backbone};
      const uint64_t* keys = at<uint64_t>(wsc, p.keys);
      int32_t* tok_c = tokens + (size_t)b0 * n;
      for (int i = 0; i < n; ++i) {
        const uint16_t* th = (i == 0) ? target_hidden + (size_t)b0 * c.backbone : hid[(i - 1) & 1];
        // step i's token: the caller's for i = 0, else the previous step's argmax (recorded as tokens[:, i-1])
        mtpd::TokenSource ts{last_token + b0, keys, 0, key_slots(c), nullptr, 0, nullptr};
        if (i > 0) ts = mtpd::TokenSource{last_token + b0, keys, 1, key_slots(c), tok_c + (i - 1), n, nullptr};
        uint16_t* hout = (i == n - 1) ? hidden_out + (size_t)b0 * c.backbone : hid[i & 1];
        CHECK(run_step(h, cs, wsc, p, Bc, th, ts, target_embd, &v.kv, v.win, v.nsplit,
                       logits ? logits + (size_t)i * BV + (size_t)b0 * c.vocab : nullptr, hout, nullptr, nullptr,
                       nullptr));
      }
      KLAUNCH(h, "final", mtpd::launch_final(cs, Bc, key_slots(c), keys, at<int32_t>(wsc, p.tok), tok_c + (n - 1), n));
      return MTPD_OK;
  });
}

int mtpd_masked_head(mtpd_handle h, void* stream, void* workspace, int32_t m, const float* hidden, float* logits,
                     int32_t* argmax, int32_t* sel_centroids, int32_t* sparse_ids, float* sparse_logits) {
  g_last_error.clear();
  CHECK(check_call(h, workspace, m));
  CHECK(check_ptr(hidden, "hidden"));
  if (!argmax) return fail(MTPD_EINVAL, "argmax is NULL");
  if (logits) CHECK(check_ptr(logits, "logits"));
  CHECK(check_head_outputs(h, sel_centroids, sparse_ids, sparse_logits));
  const Chains ch = make_chains(m);
  const Plan p = make_plan(h->cfg, ch.bmax, h->vsc);
  const mtpd_config& c = h->cfg;
  const size_t kv_n = (size_t)c.top_k * h->vsc;
  const CallKey key = make_key(3, m, 1, {workspace, hidden, logits, argmax, sel_centroids, sparse_ids, sparse_logits},
                               nullptr, nullptr, nullptr);
  return run_call(h, static_cast<hipStream_t>(stream), key, ch, [&](int ci, hipStream_t cs) -> int {
      const int b0 = ch.rows[ci], Bc = ch.rows[ci + 1] - b0;
      void* wsc = static_cast<char*>(workspace) + (size_t)ci * p.total;
      const float* hc = hidden + (size_t)b0 * c.hidden;
      float* lc = logits ? logits + (size_t)b0 * c.vocab : nullptr;
      if (c.n_centroids == 0) {  // dense tied head
        KLAUNCH(h, "zero_keys", mtpd::launch_zero_keys(cs, at<uint64_t>(wsc, p.keys), Bc));
        CHECK(run_head(h, cs, wsc, p, Bc, hc, lc, nullptr, nullptr, nullptr));
        KLAUNCH(h, "final", mtpd::launch_final(cs, Bc, 1, at<uint64_t>(wsc, p.keys), argmax + b0, nullptr, 0));
        return MTPD_OK;
      }
      // [Inventory] "Centroid / ordered embeddings LM head", step 1: centroid logits
      KLAUNCH(h, "scores", mtpd::launch_scores(cs, Bc, c.hidden, c.n_centroids, hc, h->w.centroids, at<float>(wsc, p.scores)));
      if (lc) KLAUNCH(h, "fill", mtpd::launch_fill(cs, lc, (size_t)Bc * c.vocab));
      CHECK(run_head(h, cs, wsc, p, Bc, hc, lc, sel_centroids ? sel_centroids + (size_t)b0 * c.top_k : nullptr,
                     sparse_ids ? sparse_ids + b0 * kv_n : nullptr, sparse_logits ? sparse_logits + b0 * kv_n : nullptr));
      KLAUNCH(h, "final", mtpd::launch_final(cs, Bc, c.top_k, at<uint64_t>(wsc, p.keys), argmax + b0, nullptr, 0));
      return MTPD_OK;
  });
}

}  // extern "C"

namespace {

// Sampling of the row's token from the head outputs already in the workspace (sparse logits, ids and selected
// clusters for the masked head; the logits row `dense_row` for the dense head).
int run_sample(const mtpd_handle_s* h, hipStream_t s, void* ws, const Plan& p, int B, const float* dense_row,
               float temperature, const float* u, int32_t* tok_out, float* prob_out, int out_stride) {
  const mtpd_config& c = h->cfg;
  const bool dense = c.n_centroids == 0;
  const int n = dense ? c.vocab : c.top_k * h->vsc;
  const float* vals = dense ? dense_row : at<float>(ws, p.z);
  const int k = dense ? 0 : c.top_k;
  if (n > 4096)  // several tiles: their sums first (a single tile is summed by the draw itself)
    KLAUNCH(h, "sample_tiles", mtpd::launch_sample(s, 0, B, n, h->vsc, k, vals, at<int32_t>(ws, p.ids), at<int32_t>(ws, p.sel),
                                                 at<uint64_t>(ws, p.keys), key_slots(c), temperature,
                                                 at<float>(ws, p.tsum), u, tok_out, prob_out, out_stride,
                                                 at<int32_t>(ws, p.stok)));
  KLAUNCH(h, "sample_pick", mtpd::launch_sample(s, 1, B, n, h->vsc, k, vals, at<int32_t>(ws, p.ids), at<int32_t>(ws, p.sel),
                                                at<uint64_t>(ws, p.keys), key_slots(c), temperature,
                                                at<float>(ws, p.tsum), u, tok_out, prob_out, out_stride,
                                                at<int32_t>(ws, p.stok)));
  return MTPD_OK;
}

int check_sampling(const mtpd_handle_s* h, float temperature, const float* u) {
  if (!(temperature > 0.f) || !std::isfinite(temperature)) return fail(MTPD_EINVAL, "temperature must be > 0 and finite");
  if (!u) return fail(MTPD_EINVAL, "uniforms is NULL");
  if (h->cfg.n_centroids == 0 && h->cfg.vocab > mtpd::kMaxSampleTiles * 4096)
    return fail(MTPD_EUNSUP, "sampling the dense head needs vocab <= %d", mtpd::kMaxSampleTiles * 4096);
  return MTPD_OK;
}

}  // namespace

extern "C" {

int mtpd_draft_block_sampled(mtpd_handle h, void* stream, void* workspace, int32_t batch, int32_t n,
                             const uint16_t* target_hidden, const int32_t* last_token, const uint16_t* target_embd,
                             const mtpd_shared_kv* kv, float temperature, const float* uniforms, int32_t* tokens,
                             float* probs, float* logits, uint16_t* hidden_out) {
  g_last_error.clear();
  CHECK(check_call(h, workspace, batch));
  if (n < 1 || n > 64) return fail(MTPD_ESHAPE, "n must be in [1, 64]");
  CHECK(check_sampling(h, temperature, uniforms));
  mtpd::RowWindows win[2];
  int nsplit[2];
  CHECK(check_step_inputs(h, batch, target_hidden, last_token, target_embd, kv, win, nsplit));
  if (!tokens) return fail(MTPD_EINVAL, "tokens is NULL");
  CHECK(check_ptr(hidden_out, "hidden_out"));
  if (logits) CHECK(check_ptr(logits, "logits"));
  const Chains ch = make_chains(batch);
  const Plan p = make_plan(h->cfg, ch.bmax, h->vsc);
  const mtpd_config& c = h->cfg;
  const bool dense = c.n_centroids == 0;
  const size_t BV = (size_t)batch * c.vocab;
  const CallKey key = make_key(4, batch, n,
                               {workspace, target_hidden, last_token, target_embd, kv->sliding.k, kv->sliding.v,
                                kv->full.k, kv->full.v, kv->rope, uniforms, tokens, probs, logits, hidden_out},
                               win, nsplit, kv, temperature);
  return run_call(h, static_cast<hipStream_t>(stream), key, ch, [&](int ci, hipStream_t cs) -> int {
      const int b0 = ch.rows[ci], Bc = ch.rows[ci + 1] - b0;
      void* wsc = static_cast<char*>(workspace) + (size_t)ci * p.total;
      const ChainView v = chain_view(h, kv, win, b0, Bc);
      uint16_t* hid[2] = {at<uint16_t>(wsc, p.hid), at<uint16_t>(wsc, p.hid) + (size_t)Bc * c.backbone};
      const uint64_t* keys = at<uint64_t>(wsc, p.keys);
      for (int i = 0; i < n; ++i) {
        const uint16_t* th = (i == 0) ? target_hidden + (size_t)b0 * c.backbone : hid[(i - 1) & 1];
        // step i's token: the caller's for i = 0, else the token the previous step drew
        const mtpd::TokenSource ts{i == 0 ? last_token + b0 : at<int32_t>(wsc, p.stok), keys, 0, key_slots(c),
                                   nullptr, 0, nullptr};
        uint16_t* hout = (i == n - 1) ? hidden_out + (size_t)b0 * c.backbone : hid[i & 1];
        float* lrow = logits ? logits + (size_t)i * BV + (size_t)b0 * c.vocab : (dense ? at<float>(wsc, p.row) : nullptr);
        // the masked head keeps its selected clusters, ids and sparse logits in the workspace for the sampler
        CHECK(run_step(h, cs, wsc, p, Bc, th, ts, target_embd, &v.kv, v.win, v.nsplit, lrow, hout,
                       dense ? nullptr : at<int32_t>(wsc, p.sel), dense ? nullptr : at<int32_t>(wsc, p.ids),
                       dense ? nullptr : at<float>(wsc, p.z)));
        CHECK(run_sample(h, cs, wsc, p, Bc, lrow, temperature, uniforms + (size_t)i * batch + b0,
                         tokens + (size_t)b0 * n + i, probs ? probs + (size_t)b0 * n + i : nullptr, n));
      }
      return MTPD_OK;
  });
}

int mtpd_sample_head(mtpd_handle h, void* stream, void* workspace, int32_t m, const float* hidden,
                     float temperature, const float* uniforms, int32_t* token, float* prob, float* logits) {
  g_last_error.clear();
  CHECK(check_call(h, workspace, m));
  CHECK(check_ptr(hidden, "hidden"));
  CHECK(check_sampling(h, temperature, uniforms));
  if (!token) return fail(MTPD_EINVAL, "token is NULL");
  if (logits) CHECK(check_ptr(logits, "logits"));
  const Chains ch = make_chains(m);
  const Plan p = make_plan(h->cfg, ch.bmax, h->vsc);
  const mtpd_config& c = h->cfg;
  const bool dense = c.n_centroids == 0;
  const CallKey key = make_key(5, m, 1, {workspace, hidden, uniforms, token, prob, logits}, nullptr, nullptr, nullptr,
                               temperature);
  return run_call(h, static_cast<hipStream_t>(stream), key, ch, [&](int ci, hipStream_t cs) -> int {
      const int b0 = ch.rows[ci], Bc = ch.rows[ci + 1] - b0;
      void* wsc = static_cast<char*>(workspace) + (size_t)ci * p.total;
      const float* hc = hidden + (size_t)b0 * c.hidden;
      float* lc = logits ? logits + (size_t)b0 * c.vocab : (dense ? at<float>(wsc, p.row) : nullptr);
      if (dense) {
        KLAUNCH(h, "zero_keys", mtpd::launch_zero_keys(cs, at<uint64_t>(wsc, p.keys), Bc));
        CHECK(run_head(h, cs, wsc, p, Bc, hc, lc, nullptr, nullptr, nullptr));
      } else {
        KLAUNCH(h, "scores", mtpd::launch_scores(cs, Bc, c.hidden, c.n_centroids, hc, h->w.centroids, at<float>(wsc, p.scores)));
        if (lc) KLAUNCH(h, "fill", mtpd::launch_fill(cs, lc, (size_t)Bc * c.vocab));
        CHECK(run_head(h, cs, wsc, p, Bc, hc, lc, at<int32_t>(wsc, p.sel), at<int32_t>(wsc, p.ids), at<float>(wsc, p.z)));
      }
      return run_sample(h, cs, wsc, p, Bc, lc, temperature, uniforms + b0, token + b0, prob ? prob + b0 : nullptr, 1);
  });
}

int mtpd_stream_read(const void* buf, uint64_t bytes, uint32_t key, uint32_t* sink, void* stream) {
  g_last_error.clear();
  if (!buf || (reinterpret_cast<uintptr_t>(buf) & 15)) return fail(MTPD_EINVAL, "buf is NULL or not 16-byte aligned");
  if (!sink || (reinterpret_cast<uintptr_t>(sink) & 3)) return fail(MTPD_EINVAL, "sink is NULL or misaligned");
  if (bytes % 16) return fail(MTPD_EINVAL, "bytes must be a multiple of 16");
  const hipError_t e = mtpd::launch_stream_read(static_cast<hipStream_t>(stream), buf, bytes, key, sink);
  if (e != hipSuccess) return fail(MTPD_EHIP, "stream_read: %s", hipGetErrorString(e));
  return MTPD_OK;
}

int mtpd_set_option(mtpd_handle h, int32_t option, int32_t value) {
  g_last_error.clear();
  if (!h) return fail(MTPD_EINVAL, "handle is NULL");
  switch (option) {
    case MTPD_OPT_GRAPHS:
      if (value != 0 && value != 1) return fail(MTPD_EINVAL, "MTPD_OPT_GRAPHS takes 0 or 1");
      h->use_graphs = value != 0;
      break;
    case MTPD_OPT_PERSISTENT:
      if (value != 0 && value != 1) return fail(MTPD_EINVAL, "MTPD_OPT_PERSISTENT takes 0 or 1");
      h->team_enabled = value != 0;
      break;
    case MTPD_OPT_DENSE_PATH:
      if (value < 0 || value > 2) return fail(MTPD_EINVAL, "MTPD_OPT_DENSE_PATH takes 0, 1 or 2");
      h->dense_path = value;
      break;
    case MTPD_OPT_ATTN_VALU:
      if (value != 0 && value != 1) return fail(MTPD_EINVAL, "MTPD_OPT_ATTN_VALU takes 0 or 1");
      h->attn_valu = value != 0;
      break;
    default:
      return fail(MTPD_EINVAL, "unknown option %d", option);
  }
  // captured graphs baked in the previous choice
  for (auto& e : h->graphs)
    if (e.exec) {
      (void)hipGraphExecDestroy(e.exec);
      e.exec = nullptr;
    }
  return MTPD_OK;
}

int32_t mtpd_fault_status(mtpd_handle h, int32_t clear) {
  g_last_error.clear();
  if (!h) return fail(MTPD_EINVAL, "handle is NULL");
  uint32_t st = 0;
  uint8_t* arenas[2] = {h->team_arena, static_cast<uint8_t*>(scratch_lookup())};
  for (uint8_t* ar : arenas) {
    if (!ar) continue;
    uint32_t w[2] = {0, 0};
    uint32_t* dev = reinterpret_cast<uint32_t*>(ar + mtpd::team_status_offset());
    LAUNCH(hipMemcpy(w, dev, sizeof(w), hipMemcpyDeviceToHost));
    st |= (w[0] & 0xFFu) | ((w[1] & 0xFFu) << 8);
    if (clear) LAUNCH(hipMemset(dev, 0, sizeof(w)));
  }
  return (int32_t)st;
}

#ifdef MTPD_TEAM_TRACE
// Measurement builds only: the persistent kernel's stage timeline of the last launch, [256 blocks][128] wall-clock
// ticks (100 MHz).
MTPD_API int mtpd_debug_team_trace(uint64_t* host) {
  LAUNCH(mtpd::team_trace_read(host));
  return MTPD_OK;
}
#endif

int mtpd_timing_enable(mtpd_handle h, int32_t enable) {
  g_last_error.clear();
  if (!h) return fail(MTPD_EINVAL, "handle is NULL");
  if (enable) h->n_timed = 0;
  h->timing = enable != 0;
  return MTPD_OK;
}

int32_t mtpd_timing_read(mtpd_handle h, int32_t cap, const char** names, float* ms) {
  g_last_error.clear();
  if (!h) return fail(MTPD_EINVAL, "handle is NULL");
  if (cap < 0 || (cap > 0 && (!names || !ms))) return fail(MTPD_EINVAL, "names/ms are NULL or cap < 0");
  const int32_t n = std::min(cap, h->n_timed);
  for (int32_t i = 0; i < n; ++i) {
    LAUNCH(hipEventSynchronize(h->timing_ev[2 * (size_t)i + 1]));
    float t = 0.f;
    LAUNCH(hipEventElapsedTime(&t, h->timing_ev[2 * (size_t)i], h->timing_ev[2 * (size_t)i + 1]));
    names[i] = h->timing_name[(size_t)i];
    ms[i] = t;
  }
  return h->n_timed;
}

}  // extern "C"
