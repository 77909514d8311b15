// Internal launch interface of the drafter-step kernels (gfx950). Host code in runtime.cpp sequences these on a
// stream; every launcher returns the hipError_t of its launch.
//
// Activations are fp32 throughout; stored tensors (weights, caches, embeddings, target hidden) are bf16.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mtpd {

constexpr int kMaxBatch = 64;  // rows per call (matches MTPD_MAX_BATCH)
constexpr int kMaxSplit = 32;  // key-range splits of one (row, kv head)
constexpr int kRowGroup = 4;   // batch rows handled together by the dense kernels

// Per-row key window [start, start + count) of one cache, passed by value.
struct RowWindows {
  int32_t start[kMaxBatch];
  int32_t count[kMaxBatch];
};

// Residual update applied in a dense kernel's prologue before its input norm:
//   x_new = (x_old + RMSNorm(delta; w_delta)) * scale       (delta == nullptr: x_new = x_old)
struct Residual {
  const float* x_old;       // [B][H]
  const float* delta;       // [B][H] or nullptr
  const uint16_t* w_delta;  // [H]
  float scale;
  float* x_new;             // [B][H], written by one block per row group (nullptr: not stored)
};

// Fill logits[begin, end) with -1e30 (spread over a kernel's blocks; no-op when logits is null).
struct FillRange {
  float* logits;
  size_t begin, end;
};

// x[b] = W_pre [target_hidden[b] ; escale * target_embd[tok[b]]] ; also zeroes `counters`.
hipError_t launch_pre(hipStream_t s, int B, int Bb, int H, int V, const uint16_t* th, const int32_t* tok,
                      const uint16_t* emb, float escale, const uint16_t* w_pre, float* x, uint32_t* counters,
                      int ncounters);

// q[b] = W_q RMSNorm(x_new[b]; w_norm)   (raw q, before q_norm and rotation)
hipError_t launch_qproj(hipStream_t s, int B, int H, int QD, Residual res, const uint16_t* w_norm, float eps,
                        const uint16_t* w_q, float* q);

// Split-K single-query attention with q_norm + rotation in the prologue; the last block of each (row, kv head)
// merges the splits into o[b][h*hd + d] (fp32).
hipError_t launch_attn(hipStream_t s, int B, int nh, int nkv, int hd, const float* q, const uint16_t* qnorm,
                       float eps, const float* rope, int type, const uint16_t* K, const uint16_t* V, int cap,
                       const RowWindows& win, int nsplit, float scale, float* pacc, float* pml, uint32_t* cnt,
                       float* o);

// y[b] = W X[b] for fp32 X rows of width K (o_proj: K = n_head*head_dim, down: K = ffn), N outputs.
hipError_t launch_dense(hipStream_t s, int B, int K, int N, const float* X, const uint16_t* w, float* y);

// m[b] = gelu_tanh(W_g u) * (W_u u), u = RMSNorm(x_new; w_norm); also fills a slice of the logits.
hipError_t launch_ffn(hipStream_t s, int B, int H, int F, Residual res, const uint16_t* w_norm, float eps,
                      const uint16_t* w_gate, const uint16_t* w_up, float* m, FillRange fill);

// h = RMSNorm(x_new; w_out) (stored to h_out); hidden_out = bf16(W_post h); scores = centroids h.
hipError_t launch_post(hipStream_t s, int B, int H, int Bb, int C, Residual res, const uint16_t* w_out, float eps,
                       const uint16_t* w_post, const uint16_t* w_cen, float* h_out, uint16_t* hidden_out,
                       float* scores);

// Top-k of C fp32 scores per row, descending, ties to the lower index.
hipError_t launch_topk(hipStream_t s, int B, const float* scores, int C, int k, int32_t* sel);

// Sparse head: ids = ordering[sel*vsc + t], z = token_embd[id] . h, optional scatter into logits, and the argmax
// (ties to the lowest id) written to next[b] and, if set, out2[b*stride2].
hipError_t launch_head(hipStream_t s, int B, int k, int vsc, int H, const int32_t* sel, const int32_t* ordering,
                       const uint16_t* E, const float* h, int32_t* ids, float* z, float* logits, size_t V,
                       uint64_t* keys, uint32_t* cnt, int32_t* next, int32_t* out2, int stride2);

// p[0, n) = 0
hipError_t launch_zero_u32(hipStream_t s, uint32_t* p, int n);

// logits[0, n) = -1e30
hipError_t launch_fill(hipStream_t s, float* logits, size_t n);

}  // namespace mtpd
