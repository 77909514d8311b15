/*
 * mtpd.h - C ABI of the MI355X (gfx950) drafter-step library: one draft step of the Gemma 4 assistant
 * (multi-token-prediction drafter), a block of chained steps, and the LM head: centroid-clustered (masked) or
 * dense (tied to the full embedding table).
 *
 * Pages cited (by title; sections as headed on each page):
 *   [MTP doc]    "Gemma 4 Multi-Token Prediction (MTP) drafter" (llama.cpp fork, gemma4-assistant.md)
 *   [Inventory]  "Gemma 4 Assistant (MTP drafter) - tensor inventory (Stage 0)"
 *   [Guide]      "Gemma 4 Assistant 使用指南：用 MTP 投机解码与 KV Sharing 加速 Gemma 4 推理" (gitcode blog)
 *   [Explained]  "Gemma 4 drafter explained" (techtwitter)
 *
 * Conventions for every entry point:
 *   - Tensors are DEVICE memory owned by the caller unless marked HOST. bf16 values are passed as their uint16_t
 *     bit patterns. Matrices are row-major [out][in] (the PyTorch nn.Linear layout, which is the GGUF [in, out]
 *     shape of the [MTP doc] "Tensor schema" read as ne0 = in). Device pointers must be 16-byte aligned.
 *   - Weights are borrowed by mtpd_create and must outlive the handle. The exception is the masked head's table:
 *     mtpd_create copies token_embd into cluster order (row r = token_embd[token_ordering[r]], vocab*hidden bf16
 *     of device memory owned by the handle), so later changes to token_embd or token_ordering are not seen.
 *   - Calls enqueue work on the caller's HIP stream (passed as void*, a hipStream_t; NULL = the null stream) and
 *     return without synchronising it. All argument validation happens on the host before anything is enqueued;
 *     on a negative return nothing was enqueued and mtpd_last_error() describes the problem.
 *   - The workspace (device, caller-owned, mtpd_workspace_bytes(h, batch) bytes, 256-byte aligned) holds every
 *     intermediate. Calls that share a workspace must be ordered on one stream.
 *   - Arithmetic: bf16 storage (weights, caches, embeddings, target hidden, hidden_out), fp32 activations and
 *     accumulation; top-k and argmax are taken on fp32 values (descending, ties to the lower index).
 */
#ifndef MTPD_H
#define MTPD_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__)
#define MTPD_API __attribute__((visibility("default")))
#else
#define MTPD_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

enum {
  MTPD_OK = 0,
  MTPD_EINVAL = -1, /* null required pointer, misaligned pointer, bad argument value */
  MTPD_ESHAPE = -2, /* configuration or per-call sizes violate a structural rule */
  MTPD_ENOMEM = -3, /* host or device allocation failed inside mtpd_create */
  MTPD_EHIP = -4,   /* a HIP runtime call or kernel launch failed */
  MTPD_EUNSUP = -5  /* valid per the pages but not implemented by this library */
};

#define MTPD_MAX_BATCH 256 /* rows per call */
#define MTPD_MAX_TIMED 4096 /* kernel timing records kept per handle */

typedef struct mtpd_handle_s *mtpd_handle;

/* Drafter hyper-parameters. [MTP doc] "Conversion" (backbone_hidden_size, num_centroids,
 * centroid_intermediate_top_k), "Variants supported" (4 layers, hidden 256, KV heads); [Inventory]
 * "HF config highlights" (three sliding + one full layer, attention_k_eq_v, vocab 262144).
 * Rules checked by mtpd_create: all sizes > 0 except n_centroids; n_head / n_kv_head in {1,2,4,8}; head_dim in
 * {64,128,256}; hidden, backbone, ffn, n_head*head_dim multiples of 256 (hidden <= 1024, backbone <= 8192, ffn and
 * n_head*head_dim <= 4096); n_layer <= 32.
 * Masked head (n_centroids > 0): vocab % n_centroids == 0; top_k <= min(n_centroids, 64); vocab / n_centroids a
 * multiple of 16, <= 1024; n_centroids <= 4096.
 * Dense tied head (n_centroids == 0: the use_ordered_embeddings=false form, [Guide] section 5; [MTP doc]
 * "Variants supported" for the large drafters): top_k 0 or 1 (unused); vocab a multiple of 16. */
typedef struct {
  int32_t backbone;          /* target model width (1536 E2B, 2560 E4B) */
  int32_t hidden;            /* drafter width (256) */
  int32_t n_layer;           /* decoder layers (4) */
  int32_t n_head;            /* query heads per layer */
  int32_t n_kv_head;         /* heads of the shared cache */
  int32_t head_dim;
  int32_t ffn;               /* GeGLU intermediate width */
  int32_t vocab;
  int32_t n_centroids;       /* clusters of the masked head (2048); 0 selects the dense tied head */
  int32_t top_k;             /* clusters kept (32) */
  int32_t swa_window;        /* keys read by a sliding layer */
  uint32_t full_attn_layers; /* bit l set: layer l reads the full-attention cache, else the sliding one */
  float rms_eps;
  float attn_scale;          /* softmax scale applied to q.k */
  float embed_scale;         /* factor on the embedded token before pre_projection (1.0) */
} mtpd_config;

/* Per-layer weights, names as in [MTP doc] "Tensor schema" (blk.{i}.*). Shapes row-major:
 * attn_q [n_head*head_dim][hidden], attn_q_norm [head_dim], attn_output [hidden][n_head*head_dim],
 * attn_norm / post_attention_norm / ffn_norm / post_ffw_norm [hidden], ffn_gate / ffn_up [ffn][hidden],
 * ffn_down [hidden][ffn]. layer_output_scale is the layer's scalar gate ([MTP doc] "What it is"), passed by value. */
typedef struct {
  const uint16_t *attn_q, *attn_q_norm, *attn_output, *attn_norm, *post_attention_norm;
  const uint16_t *ffn_norm, *post_ffw_norm, *ffn_gate, *ffn_up, *ffn_down;
  float layer_output_scale;
} mtpd_layer;

/* Global weights ([MTP doc] "Tensor schema"; [Inventory] "Expected safetensors names"):
 * pre_proj [hidden][2*backbone] (input = [target hidden ; token embedding]), post_proj [backbone][hidden],
 * output_norm [hidden], token_embd [vocab][hidden] (the head table), centroids [n_centroids][hidden],
 * token_ordering [vocab] int32, a permutation of the vocabulary viewed as [n_centroids][vocab/n_centroids]
 * ([Inventory] "Centroid / ordered embeddings LM head", step 3). centroids and token_ordering are not read (may
 * be NULL) with the dense head. layers is a HOST array [n_layer]. */
typedef struct {
  const uint16_t *pre_proj, *post_proj, *output_norm, *token_embd, *centroids;
  const int32_t *token_ordering;
  const mtpd_layer *layers;
} mtpd_weights;

/* One shared cache of the target ([MTP doc] "Runtime implementation", piece 1; [Guide] section 2(4),
 * shared_kv_states): k, v [batch][n_kv_head][cap][head_dim] bf16; v may equal k (K = V, [Inventory]
 * "Notes for llama.cpp port" 2), in which case it is read once. shared != 0: k, v are one cache
 * [1][n_kv_head][cap][head_dim] read by every row (rows of one sequence scored together, each with its own length,
 * token and position). len is a HOST array [batch], 1 <= len[b] <= cap.
 * first is an optional HOST array [batch] (NULL = all zero), 0 <= first[b] < cap: row b's valid keys, oldest
 * first, are the slots (first[b] + i) mod cap for i < len[b]. A left-padded batch ([Guide] section 2,
 * "create_attention_masks" and padding_side="left") passes its padding widths; a ring-buffer cache passes the
 * slot of its oldest key. */
typedef struct {
  const uint16_t *k, *v;
  int32_t cap;
  int32_t shared;
  const int32_t *len;
  const int32_t *first;
} mtpd_kv;

/* The two caches a drafter layer can read, plus the rotary tables for each row's constant position
 * ([Guide] section 2(2)): rope [batch][2 (0 sliding, 1 full)][2 (cos, sin)][head_dim/2] fp32, device. */
typedef struct {
  mtpd_kv sliding, full;
  const float *rope;
} mtpd_shared_kv;

/* Validate the configuration and weights and build a handle. With the masked head, copies token_ordering to the
 * host once (a blocking copy on the null stream) to check that it is a permutation ([Inventory] "GGUF /
 * converter layout", verification script), then builds the cluster-ordered head table on the null stream and
 * waits for it (MTPD_ENOMEM if it does not fit); the dense head reads token_embd as given and allocates nothing.
 * max_batch <= MTPD_MAX_BATCH. Returns MTPD_OK and *out, or a negative code. */
MTPD_API int mtpd_create(const mtpd_config *cfg, const mtpd_weights *w, int32_t max_batch, mtpd_handle *out);

/* Release a handle (NULL is a no-op). Does not touch caller memory. */
MTPD_API void mtpd_destroy(mtpd_handle h);

/* Bytes of workspace needed for calls with `batch` rows (0 on a bad handle or batch). */
MTPD_API size_t mtpd_workspace_bytes(mtpd_handle h, int32_t batch);

/* One drafter step for `batch` independent rows ([MTP doc] "What it is"; [Guide] sections 2 and 6;
 * [Explained] "Target Activations", "KV Cache Sharing", "The Efficient Embedder"):
 *   x = pre_proj [target_hidden[b] ; embed_scale * target_embd[last_token[b]]]
 *   4 Q-only layers over the shared caches (sliding layers: the last min(window, len) keys; full: all len keys)
 *   h = output_norm(x); hidden_out = post_proj h (bf16)
 *   masked head: top_k of centroids.h, their vocab/n_centroids token ids through token_ordering, sparse logits
 *   token_embd[id].h, a -1e30 row with the sparse logits scattered in, next_token = argmax;
 *   dense head: the row is token_embd[v].h for every v, next_token = argmax (ties to the lowest id).
 * target_hidden [batch][backbone] bf16; last_token [batch] int32 in [0, vocab) (out-of-range ids are clamped
 * into range); target_embd [vocab][backbone] bf16 (the target's input embedding table).
 * Outputs: next_token [batch] int32, hidden_out [batch][backbone] bf16 (required); logits [batch][vocab] fp32,
 * sel_centroids [batch][top_k] int32 (descending score), sparse_ids / sparse_logits [batch][top_k*vsc]
 * (optional, NULL to skip; the last three must be NULL with the dense head: MTPD_EINVAL otherwise). */
MTPD_API int mtpd_drafter_step(mtpd_handle h, void *stream, void *workspace, int32_t batch, const uint16_t *target_hidden,
                      const int32_t *last_token, const uint16_t *target_embd, const mtpd_shared_kv *kv,
                      float *logits, int32_t *next_token, uint16_t *hidden_out, int32_t *sel_centroids,
                      int32_t *sparse_ids, float *sparse_logits);

/* mtpd_drafter_step without a workspace argument and without any allocation during the call, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving loops, and harnesses that forbid
 * hipMalloc. Arguments, outputs and results are those of mtpd_drafter_step. The intermediates live in a
 * file-scope device array of the library (MTPD_NOALLOC_SCRATCH_BYTES, one copy per device, resolved by the first
 * mtpd_create on that device and held until the process ends). Batches whose workspace (mtpd_workspace_bytes)
 * exceeds that size are rejected with MTPD_ESHAPE before anything is enqueued; MTPD_EINVAL if no handle was ever
 * created on the current device. The kernels are launched directly on `stream` (no graph is instantiated) and no
 * timing records are taken. Every call on one device shares that array and it keeps the last call's contents: calls
 * that overlap on one device (different streams, or different threads without ordering) race and must not be
 * issued. */
#define MTPD_NOALLOC_SCRATCH_BYTES (8u << 20)
MTPD_API int mtpd_drafter_step_noalloc(mtpd_handle h, void *stream, int32_t batch, const uint16_t *target_hidden,
                      const int32_t *last_token, const uint16_t *target_embd, const mtpd_shared_kv *kv,
                      float *logits, int32_t *next_token, uint16_t *hidden_out, int32_t *sel_centroids,
                      int32_t *sparse_ids, float *sparse_logits);

/* n >= 1 chained drafter steps at the constant position over the same caches ([Guide] section 2(3): within a
 * draft round the last-seen token is the drafter's own; [Explained] "Target Activations": later rounds take the
 * drafter's own post-projected activations). Step i+1 reads step i's hidden_out and next token on the device.
 * tokens [batch][n] int32 (required); logits [n][batch][vocab] fp32 (optional); hidden_out [batch][backbone]
 * bf16 of the last step (required). */
MTPD_API int mtpd_draft_block(mtpd_handle h, void *stream, void *workspace, int32_t batch, int32_t n,
                     const uint16_t *target_hidden, const int32_t *last_token, const uint16_t *target_embd,
                     const mtpd_shared_kv *kv, int32_t *tokens, float *logits, uint16_t *hidden_out);

/* The masked head alone on m rows of fp32 hidden states h [m][hidden] (normed, as the head receives them):
 * [Inventory] "Centroid / ordered embeddings LM head" steps 1-5. argmax [m] int32 required; logits [m][vocab],
 * sel_centroids [m][top_k], sparse_ids / sparse_logits [m][top_k*vsc] optional. m <= max_batch.
 * With n_centroids == 0 this is the dense tied head: logits [m][vocab] = token_embd . h (optional), argmax; the
 * per-cluster outputs must be NULL. */
MTPD_API int mtpd_masked_head(mtpd_handle h, void *stream, void *workspace, int32_t m, const float *hidden,
                     float *logits, int32_t *argmax, int32_t *sel_centroids, int32_t *sparse_ids,
                     float *sparse_logits);

/* draft_block(n) with sampled tokens instead of the argmax, for stochastic acceptance ([MTP doc] "Runtime
 * implementation (shipped)": the accept rate varies with temperature; [Inventory] "Centroid / ordered embeddings LM
 * head", step 5: the full logits row exists for sampling). Step i draws its token from p = softmax(row / temperature)
 * over the row's scored tokens (the masked head's top_k * vsc candidates, or the whole vocabulary with the dense
 * head; masked entries have p = 0) by inverse CDF at uniforms[i][b], the CDF running in the head table's row order:
 * the selected clusters by ascending cluster index, each cluster's ids in token_ordering order (dense head: token
 * order). Step i+1 reads that token. temperature > 0 and finite; uniforms [n][batch] fp32 device, in [0, 1) (u >= 1
 * draws the last token with p > 0). tokens [batch][n] int32 (required); probs [batch][n] fp32, the draft
 * probability of each drawn token (optional); logits [n][batch][vocab] (optional); hidden_out as draft_block.
 * With the dense head, vocab <= 1048576 (MTPD_EUNSUP otherwise). */
MTPD_API int mtpd_draft_block_sampled(mtpd_handle h, void *stream, void *workspace, int32_t batch, int32_t n,
                     const uint16_t *target_hidden, const int32_t *last_token, const uint16_t *target_embd,
                     const mtpd_shared_kv *kv, float temperature, const float *uniforms, int32_t *tokens,
                     float *probs, float *logits, uint16_t *hidden_out);

/* The head alone with a sampled token: m rows of fp32 normed states h [m][hidden], one token per row drawn as in
 * mtpd_draft_block_sampled at uniforms[b] ([m] device). token [m] int32 (required); prob [m] (optional); logits
 * [m][vocab] (optional: the masked head's -1e30 row, or the dense row). */
MTPD_API int mtpd_sample_head(mtpd_handle h, void *stream, void *workspace, int32_t m, const float *hidden,
                     float temperature, const float *uniforms, int32_t *token, float *prob, float *logits);

/* Handle options (set after mtpd_create; each change discards the handle's captured graphs). Values:
 *   MTPD_OPT_GRAPHS      1 (default): replay each call from a captured HIP graph; 0: launch every kernel directly.
 *   MTPD_OPT_PERSISTENT  1 (default): calls of at most 16 rows on per-row K = V caches of the E2B / E4B shapes
 *                        (hidden 256, 4 heads of 256 over one or two kv heads, FFN 1024, 2048 clusters of 128, top
 *                        32, <= 4 layers) on a 256-CU gfx950 run as one launch of the persistent drafter kernel, whose blocks
 *                        hand values to each other inside each XCD; it needs every CU free for the launch (a wait
 *                        that cannot finish gives up after a bounded time and is reported by mtpd_fault_status).
 *                        0: the per-stage kernels.
 *   MTPD_OPT_DENSE_PATH  0 (default): dense stages by batch size (fused small-batch kernels below 32 rows, matrix-core
 *                        GEMMs from 32 rows); 1: always the small-batch kernels; 2: always the GEMMs. A backbone
 *                        above 4096 always runs the small-batch kernels (the GEMMs reduce over at most 8192).
 *   MTPD_OPT_ATTN_VALU   0 (default); 1: the vector-ALU attention kernel for every shape.
 * Returns MTPD_OK or MTPD_EINVAL (unknown option or value). */
enum { MTPD_OPT_GRAPHS = 1, MTPD_OPT_PERSISTENT = 2, MTPD_OPT_DENSE_PATH = 3, MTPD_OPT_ATTN_VALU = 4 };
MTPD_API int mtpd_set_option(mtpd_handle h, int32_t option, int32_t value);

/* Status of the persistent drafter kernel's launches on this handle and on the allocation-free entry point's scratch
 * of the current device: 0 if every launch so far finished its waits normally, else bit 0 (a wait gave up, the
 * launch's outputs are undefined), bit 1 (a block ran on an XCD outside the 8 the kernel expects) and in bits 8-15
 * one plus the largest stage id among the waits that gave up. Waits for the device (a blocking copy); clear != 0
 * resets the status. */
MTPD_API int32_t mtpd_fault_status(mtpd_handle h, int32_t clear);

/* Kernel timing, a measurement aid outside the method. While enabled on a handle, drafter_step, draft_block and
 * masked_head launch their kernels directly on the caller's stream (captured graphs are not replayed) and attach
 * to each launch a pair of HIP events that the runtime records at the kernel's start and end. Enabling clears
 * the records; disabling keeps them for reading; at most MTPD_MAX_TIMED launches are recorded, later ones are not.
 * Not thread-safe per handle. Returns MTPD_OK or MTPD_EINVAL. */
MTPD_API int mtpd_timing_enable(mtpd_handle h, int32_t enable);

/* Waits for the recorded events and copies min(cap, count) records in launch order: names[i] is a static label of
 * the launch site ("pre", "qproj", "attn_sliding", "attn_full", "attn_merge_sliding", "attn_merge_full",
 * "o_proj", "ffn", "down", "post", "head", "head_dense", "zero_keys", "final", "scores", "fill", "sample_tiles", "sample_pick"), ms[i] its
 * duration in milliseconds.
 * names and ms are caller-owned host arrays of cap entries. Returns the number of records (which may exceed cap)
 * or a negative error code. */
MTPD_API int32_t mtpd_timing_read(mtpd_handle h, int32_t cap, const char **names, float *ms);

/* Streaming read, a measurement aid outside the method: reads `bytes` at buf (device memory, 16-byte aligned,
 * bytes a multiple of 16) with 16-byte vector loads spread over every CU, enqueued on `stream`, and writes nothing
 * but possibly sink[0] (a caller-owned device word, written only if the xor of every word read equals `key`). One
 * call over a buffer much larger than the last-level caches (1 GiB against 8 x 4 MB L2 and the 256 MB memory-side
 * cache) measures the sustained read rate and leaves the caches holding that buffer's clean lines.
 * Returns MTPD_OK, MTPD_EINVAL (NULL or misaligned pointer, bytes not a multiple of 16) or MTPD_EHIP. */
MTPD_API int mtpd_stream_read(const void *buf, uint64_t bytes, uint32_t key, uint32_t *sink, void *stream);

/* Message for the last non-OK return on the calling thread ("" if none). */
MTPD_API const char *mtpd_last_error(void);

/* ABI version: 6 (mtpd_kv gained `first` in 2 and `shared` in 3; mtpd_drafter_step_noalloc in 4; options and
 * the persistent kernel's status in 5; mtpd_stream_read in 6). */
MTPD_API int32_t mtpd_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MTPD_H */
