// LM heads: the centroid-masked head (top-k of centroid scores, gathered cluster rows, sparse logits, scatter and
// argmax keys), the dense tied head, the cluster-order table build, the final argmax and the -1e30 fill.
//
// Pages cited (by title; sections as headed on each page):
//   [MTP doc]    "Gemma 4 Multi-Token Prediction (MTP) drafter" (llama.cpp fork, gemma4-assistant.md)
//   [Inventory]  "Gemma 4 Assistant (MTP drafter) - tensor inventory (Stage 0)"
//   [Guide]      "Gemma 4 Assistant 使用指南：用 MTP 投机解码与 KV Sharing 加速 Gemma 4 推理" (gitcode blog)
#include "device.h"

namespace mtpd {
namespace {

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
  __shared__ uint32_t sh_n;
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
  // than one after all four passes) need ordering by index, below. Each wave counts into its own histogram and
  // every wave scans all four after the pass's one barrier (so the chosen digit never goes through LDS); a wave
  // then clears its own histogram of the other buffer, last read before this pass's barrier, for the next pass.
  uint32_t prefix = 0, pmask = 0;
  uint32_t need = (uint32_t)j + 1u;
  uint32_t inbin = 0;
#pragma unroll
  for (int q2 = 0; q2 < 4; ++q2) hist[0][wave][lane + 64 * q2] = hist[1][wave][lane + 64 * q2] = 0u;
  int buf = 0;
  for (int shift = 24; shift >= 0; shift -= 8) {
#pragma unroll
    for (int i = 0; i < NPT; ++i)
      if (tid + 256 * i < C && (ok[i] & pmask) == prefix)
        atomicAdd(&hist[buf][wave][(ok[i] >> shift) & 255u], 1u);
    __syncthreads();
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
    uint32_t before = incl - sum, dsel = 0u, bsel = 0u, nsel = 0u;
    bool hit = false;
#pragma unroll
    for (int q2 = 0; q2 < 4; ++q2) {
      if (before < need && before + cnt[q2] >= need) {
        hit = true;
        dsel = 255u - 4u * lane - q2;
        bsel = before;
        nsel = cnt[q2];
      }
      before += cnt[q2];
    }
    const uint64_t hm = __ballot(hit);  // exactly one lane: the bins partition the ranks 1 .. (bin size)
    const int src = hm ? __ffsll((unsigned long long)hm) - 1 : 0;
    const uint32_t digit = (uint32_t)__builtin_amdgcn_readlane((int)dsel, src);
    const uint32_t nbefore = (uint32_t)__builtin_amdgcn_readlane((int)bsel, src);
    inbin = (uint32_t)__builtin_amdgcn_readlane((int)nsel, src);
#pragma unroll
    for (int q2 = 0; q2 < 4; ++q2) hist[buf ^ 1][wave][lane + 64 * q2] = 0u;
    prefix |= digit << shift;
    pmask |= 255u << shift;
    need -= nbefore;
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
    uint32_t hi[2], lo[2];
    split_bf16x2(live ? f[0] : 0.f, live ? f[1] : 0.f, hi[0], lo[0]);
    split_bf16x2(live ? f[2] : 0.f, live ? f[3] : 0.f, hi[1], lo[1]);
    *reinterpret_cast<uint2*>(&hs[0][col][k]) = make_uint2(hi[0], hi[1]);
    *reinterpret_cast<uint2*>(&hs[1][col][k]) = make_uint2(lo[0], lo[1]);
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
            // streaming stores: the row is not read again here, and dirty lines left in L2 would be written back
            // during the next kernels
            __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(logits + (size_t)col * V + row0));
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

// ------------------------------------------------------------------------------------------------------------
// Cluster-grouped scoring for many rows ([Inventory] "Centroid / ordered embeddings LM head", steps 3-5, the same
// outputs as k_head): when the batch's rows select many clusters in common, each selected cluster's rows are read
// once and scored for every (row, slot) that selected it.
//
// k_topk_rows (one block of 256 threads per row): the row's top k centroids in slot order (descending score, ties
// to the lower index); sel[b][j] = slot j's centroid. A radix select on the order keys, 8 bits at a time from the
// top, finds the bin that holds the k-th element. Elements in higher bins (fewer than k) take the first slots by
// their rank among themselves; the bin's members, all tied at the resolved bits (or the bin's only member when the
// search stopped early), take the remaining slots in ascending index order.
template <int NPT>
__global__ __launch_bounds__(256) void k_topk_rows(int C, int k, const float* scores, int32_t* sel) {
  __shared__ uint32_t hist[2][4][256];
  __shared__ uint32_t sh_digit, sh_before, sh_n, sh_above;
  __shared__ uint64_t above[kMaxTopK];
  __shared__ uint32_t bcount[NPT][4];
  const int b = blockIdx.x, tid = threadIdx.x, lane = lane_id(), wave = wave_id();
  uint32_t ok[NPT];
#pragma unroll
  for (int i = 0; i < NPT; ++i) ok[i] = f32_order(scores[(size_t)b * C + min(tid + 256 * i, C - 1)]);
  uint32_t prefix = 0, pmask = 0, need = (uint32_t)k, inbin = 0;
  hist[0][0][tid] = hist[0][1][tid] = hist[0][2][tid] = hist[0][3][tid] = 0u;
  if (tid == 0) sh_above = 0u;
  __syncthreads();
  int buf = 0;
  for (int shift = 24; shift >= 0; shift -= 8) {
#pragma unroll
    for (int i = 0; i < NPT; ++i)
      if (tid + 256 * i < C && (ok[i] & pmask) == prefix) atomicAdd(&hist[buf][wave][(ok[i] >> shift) & 255u], 1u);
    __syncthreads();
    if (wave == 0) {
      uint32_t cnt[4], sum = 0;  // lane l owns digits 255-4l .. 252-4l (descending)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int dg = 255 - 4 * lane - q;
        cnt[q] = hist[buf][0][dg] + hist[buf][1][dg] + hist[buf][2][dg] + hist[buf][3][dg];
        sum += cnt[q];
      }
      uint32_t incl = sum;
#pragma unroll
      for (int of = 1; of < 64; of <<= 1) {
        const uint32_t t = __shfl_up(incl, of, 64);
        if (lane >= of) incl += t;
      }
      uint32_t before = incl - sum;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (before < need && before + cnt[q] >= need) {
          sh_digit = 255u - 4u * lane - q;
          sh_before = before;
          sh_n = cnt[q];
        }
        before += cnt[q];
      }
    } else {
      for (int i = (wave - 1) * 64 + lane; i < 4 * 256; i += 3 * 64) (&hist[buf ^ 1][0][0])[i] = 0u;
    }
    __syncthreads();
    prefix |= sh_digit << shift;
    pmask |= 255u << shift;
    need -= sh_before;
    inbin = sh_n;
    buf ^= 1;
    if (inbin == 1u) break;
  }
  const uint32_t nabove = (uint32_t)k - need;  // elements in higher bins: fewer than k <= 64
  // bin members: their rank in index order (index tid + 256 i runs i-major, then wave, then lane)
  uint64_t inb[NPT];
#pragma unroll
  for (int i = 0; i < NPT; ++i) {
    const bool mem = tid + 256 * i < C && (ok[i] & pmask) == prefix;
    inb[i] = __ballot(mem);
    if (lane == 0) bcount[i][wave] = (uint32_t)__popcll(inb[i]);
    if (tid + 256 * i < C && (ok[i] & pmask) > prefix) {
      const uint32_t pos = atomicAdd(&sh_above, 1u);
      above[pos] = ((uint64_t)ok[i] << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)(tid + 256 * i));
    }
  }
  __syncthreads();
  uint32_t base = 0;
#pragma unroll
  for (int i = 0; i < NPT; ++i) {
    uint32_t r = base;
    for (int w = 0; w < wave; ++w) r += bcount[i][w];
    r += (uint32_t)__popcll(inb[i] & ((1ull << lane) - 1ull));
    if (((inb[i] >> lane) & 1ull) && r < need) sel[(size_t)b * k + nabove + r] = tid + 256 * i;
    base += bcount[i][0] + bcount[i][1] + bcount[i][2] + bcount[i][3];
  }
  if (wave == 0) {
    // lane e holds element e of the higher bins; its slot is the number of larger ones (distinct composites)
    const uint64_t v = (uint32_t)lane < nabove ? above[lane] : 0ull;
    const int vhi = (int)(v >> 32), vlo = (int)(uint32_t)v;
    uint32_t rank = 0;
#pragma unroll
    for (int f = 0; f < 64; ++f) {
      const uint64_t o = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane(vhi, f) << 32) |
                         (uint32_t)__builtin_amdgcn_readlane(vlo, f);
      rank += (o > v) ? 1u : 0u;
    }
    if ((uint32_t)lane < nabove) sel[(size_t)b * k + rank] = key_id(v);
  }
}

// entries of one cluster scored by one block of k_head_grouped (four 16-row matrix-core tiles)
constexpr int kGroupTile = 64;

// k_group (one block of 1024 threads): the n = B k selections sel[] grouped by cluster with a counting sort in LDS:
// a cluster's count, a "selected" flag and its number of kGroupTile-entry tiles packed in one 64-bit word go through one
// prefix scan, giving each cluster its first entry and each selected cluster its place in the compacted list and
// its first tile. Outputs: trec[T] (per tile: cluster, first entry, entry count; count 0 past the last tile, T = the
// most tiles there can be), entries[n] (flat (row, slot) indices grouped by cluster; the order inside a group does
// not matter, every entry's outputs are its own).
__global__ __launch_bounds__(1024) void k_group(int n, int C, int T, const int32_t* sel, int4* trec, int32_t* entries) {
  constexpr int EPT = kMaxBatch * kMaxTopK / 1024;  // entries per thread at most
  constexpr int CPT = kMaxCentroids / 1024;         // clusters per thread
  __shared__ uint32_t cnt[kMaxCentroids];
  __shared__ uint64_t wtot[16];
  const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
  for (int c = tid; c < kMaxCentroids; c += 1024) cnt[c] = 0u;
  __syncthreads();
  // every selection loaded first (clamped index, unconditionally) so the loads issue together, then counted
  int cv[EPT];
  uint32_t pos[EPT];
#pragma unroll
  for (int i = 0; i < EPT; ++i) cv[i] = sel[min(tid + 1024 * i, n - 1)];
#pragma unroll
  for (int i = 0; i < EPT; ++i) {
    if (tid + 1024 * i >= n) cv[i] = -1;
    pos[i] = cv[i] >= 0 ? atomicAdd(&cnt[cv[i]], 1u) : 0u;
  }
  __syncthreads();
  // packed (tiles << 32 | flag << 16 | count) per cluster (count <= 16384, flags <= 4096, tiles <= 4352), thread-local
  // prefix over CPT consecutive clusters
  uint64_t loc[CPT], run = 0;
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c = tid * CPT + i;
    const uint32_t v = c < C ? cnt[c] : 0u;
    loc[i] = run;
    run += ((uint64_t)((v + kGroupTile - 1) / kGroupTile) << 32) | (v ? 0x10000u : 0u) | v;
  }
  uint64_t incl = run;
#pragma unroll
  for (int of = 1; of < 64; of <<= 1) {
    const uint32_t tlo = __shfl_up((uint32_t)incl, of, 64), thi = __shfl_up((uint32_t)(incl >> 32), of, 64);
    if (lane >= of) incl += ((uint64_t)thi << 32) | tlo;
  }
  if (lane == 63) wtot[wave] = incl;
  __syncthreads();
  uint64_t base = 0;
  for (int w = 0; w < wave; ++w) base += wtot[w];
  base += incl - run;
  __shared__ int ntiles;
  if (tid == 1023) ntiles = (int)((base + run) >> 32);
  __syncthreads();
  for (int t = ntiles + tid; t < T; t += 1024) trec[t] = make_int4(0, 0, 0, 0);  // no tile
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c = tid * CPT + i;
    const uint64_t pre = base + loc[i];
    if (c < C && cnt[c]) {
      const int first = (int)(pre & 0xFFFFu), t0 = (int)(pre >> 32), v = (int)cnt[c];
      for (int t = 0; t * kGroupTile < v; ++t)
        trec[t0 + t] = make_int4(c, first + t * kGroupTile, min(kGroupTile, v - t * kGroupTile), 0);
    }
    cnt[c] = (uint32_t)(pre & 0xFFFFu);  // first entry of cluster c (reused as the offset table)
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < EPT; ++i)
    if (cv[i] >= 0) entries[cnt[cv[i]] + pos[i]] = tid + 1024 * i;
}

// One block per (selected cluster, tile of up to kGroupTile of the entries that selected it) (grid = the most tiles
// there can be; blocks past the last tile exit): the cluster's vsc rows are scored against the h of the tile's
// entries (row, slot) as a matrix-core product Z[entries][ids] = H[entries][dims] . E_c[ids][dims]^T with
// v_mfma_f32_16x16x32_bf16, 16 entries at a time. A cluster chosen by many rows is thus spread over a few blocks,
// so no block carries a long tail, while most clusters are read once.
//   B operand (ids as columns): the cluster's rows, 16 ids per tile, each wave holding CTW tiles in registers
//     (lane: id 16 tile + l % 16, dims 32 s + 8 (l / 16) .. +8), loaded straight from the cluster-ordered table;
//   A operand (entries as rows): 16 entries' h, staged in LDS as bf16 hi + lo (fp32-level products);
//   D: lane l holds entries 4 (l / 16) + i, id 16 tile + l % 16.
// The epilogue writes each entry's ids, sparse logits and logits-row scatter as k_head does, and the entry's best
// (value, id) key: a 16-lane reduction, then a maximum over id tiles and waves in LDS. 256 threads, H = 128 HCH.
template <int HCH>
__global__ __launch_bounds__(256) void k_head_grouped(int k, int vsc, const int32_t* ordering, const uint16_t* Es,
                                                      const float* h, const int4* trec, const int32_t* entries,
                                                      int32_t* __restrict__ ids, float* __restrict__ z,
                                                      float* __restrict__ logits, size_t V,
                                                      uint64_t* __restrict__ keys) {
  constexpr int H = HCH * 128, KSTEPS = H / 32, LROW = H + 8;
  constexpr int CTW = HCH <= 4 ? 2 : 1;  // id tiles per wave held at once
  __shared__ unsigned long long best[kGroupTile];
  __shared__ __attribute__((aligned(16))) uint16_t hs[2][16][LROW];  // [hi / lo][entry][dim]
  const int4 rec = trec[blockIdx.x];
  const int c = rec.x, e0 = rec.y, ne = rec.z;
  if (ne == 0) return;  // block-uniform: no tile
  const int tid = threadIdx.x, lane = lane_id(), wave = wave_id();
  const int n = lane & 15, kq = lane >> 4;
  const int ct = vsc / 16;  // id tiles of the cluster
  const bool one_group = ct <= 4 * CTW;  // every id tile in registers at once
  const int32_t* ord = ordering + (size_t)c * vsc;
  const uint16_t* crow = Es + (size_t)c * vsc * H;
  if (tid < kGroupTile) best[tid] = 0ull;
  uint4 eb[CTW][KSTEPS];
  int idv[CTW];
  auto load_rows = [&](int g0) {
#pragma unroll
    for (int j = 0; j < CTW; ++j) {
      const int t = min((g0 + wave * CTW + j) * 16 + n, vsc - 1);  // the lane's id position (clamped)
#pragma unroll
      for (int s2 = 0; s2 < KSTEPS; ++s2) eb[j][s2] = ld_global16(crow + (size_t)t * H + 32 * s2 + 8 * kq);
      idv[j] = ord[t];
    }
  };
  load_rows(0);  // in flight while the first entries' h is staged

  for (int et = 0; et < ne; et += 16) {  // block-uniform: 16 entries at a time
    // every load of the tile is issued before any is used (clamped indices, no branches around the loads): the
    // entries of the thread's staged rows and of its output rows, then the staged rows of h
    constexpr int NLD = 16 * H / 4 / 256;  // float4 of h per thread
    int fl[NLD], fo[4];
#pragma unroll
    for (int q = 0; q < NLD; ++q) fl[q] = entries[e0 + min(et + (tid + 256 * q) / (H / 4), ne - 1)];
#pragma unroll
    for (int i = 0; i < 4; ++i) fo[i] = entries[e0 + min(et + 4 * kq + i, ne - 1)];
    float4 xv[NLD];
#pragma unroll
    for (int q = 0; q < NLD; ++q)
      xv[q] = *reinterpret_cast<const float4*>(h + (size_t)(fl[q] / k) * H + ((tid + 256 * q) % (H / 4)) * 4);
    __syncthreads();  // the previous tile's reads of hs (and best's initialisation) are done
#pragma unroll
    for (int q = 0; q < NLD; ++q) {
      const int i = tid + 256 * q, r = i / (H / 4), d = (i % (H / 4)) * 4;
      const bool live = et + r < ne;
      const float f[4] = {live ? xv[q].x : 0.f, live ? xv[q].y : 0.f, live ? xv[q].z : 0.f, live ? xv[q].w : 0.f};
      uint32_t hi2[2], lo2[2];
      split_bf16x2(f[0], f[1], hi2[0], lo2[0]);
      split_bf16x2(f[2], f[3], hi2[1], lo2[1]);
      *reinterpret_cast<uint2*>(&hs[0][r][d]) = make_uint2(hi2[0], hi2[1]);
      *reinterpret_cast<uint2*>(&hs[1][r][d]) = make_uint2(lo2[0], lo2[1]);
    }
    __syncthreads();

    for (int g0 = 0; g0 < ct; g0 += 4 * CTW) {  // block-uniform: groups of id tiles
      if (!one_group) load_rows(g0);
#pragma unroll
      for (int j = 0; j < CTW; ++j) {
        const int tile = g0 + wave * CTW + j;
        if (tile >= ct) break;  // wave-uniform
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s2 = 0; s2 < KSTEPS; ++s2) {
          const uint4 ah = *reinterpret_cast<const uint4*>(&hs[0][n][32 * s2 + 8 * kq]);
          const uint4 al = *reinterpret_cast<const uint4*>(&hs[1][n][32 * s2 + 8 * kq]);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ah), __builtin_bit_cast(bf16x8, eb[j][s2]), acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, al), __builtin_bit_cast(bf16x8, eb[j][s2]), acc, 0, 0, 0);
        }
        const int t = tile * 16 + n;  // id position in the cluster (< vsc: vsc is a multiple of 16)
        const uint32_t id = (uint32_t)idv[j];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int e = et + 4 * kq + i;
          uint64_t kv = 0ull;
          if (e < ne) {
            const int flat = fo[i];
            const size_t slot = (size_t)flat * vsc + t;
            if (ids) ids[slot] = (int32_t)id;
            if (z) z[slot] = acc[i];
            if (logits) logits[(size_t)(flat / k) * V + id] = acc[i];
            kv = vid_key(acc[i], id);
          }
          // maximum over the 16 ids of this tile (lanes of equal kq)
#pragma unroll
          for (int o = 8; o > 0; o >>= 1) {
            const uint32_t klo = __shfl_xor((uint32_t)kv, o, 64), khi = __shfl_xor((uint32_t)(kv >> 32), o, 64);
            kv = u64_max(kv, ((uint64_t)khi << 32) | klo);
          }
          if (n == 0 && e < ne) atomicMax(&best[e], (unsigned long long)kv);
        }
      }
    }
  }
  __syncthreads();
  if (tid < ne) keys[entries[e0 + tid]] = best[tid];
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

// ------------------------------------------------------------------------------------------------------------
// temperature sampling: p = softmax(row / T) over the scored tokens, one token per row drawn by inverse CDF at the
// caller's uniform u, the CDF running in the head table's row order (masked head: the selected clusters by ascending
// cluster index, each cluster's ids in ordering order; dense head: token order). e = 2^((v - M) * log2(e) / T) with
// M the row maximum, read from the argmax keys. The ordered elements are cut into tiles of 4096:
//   k_sample_tiles: one block per (tile, row) sums its tile's e (fixed reduction order);
//   k_sample_pick:  one block per row walks the tile sums to the tile holding u * S (S = their total), scans that
//                   tile's e in order and takes the first element whose running sum exceeds u * S.
// Both recompute e with the same instructions, so the walk and the scan see the same values.

constexpr int kSampleThreads = 1024, kSampleTile = 4 * kSampleThreads;

// Per-row setup shared by both kernels: the row maximum (into sh_M) and, for the masked head, the slot holding each
// rank of the selected clusters' ascending order (into rank2slot).
template <bool SPARSE>
__device__ __forceinline__ void sample_setup(int b, int k, const int32_t* sel, const uint64_t* keys, int nk,
                                             float* sh_M, int* rank2slot) {
  __shared__ int sel_s[kMaxTopK];
  const int wave = wave_id(), lane = lane_id(), tid = threadIdx.x;
  // both loads of wave 0 go out before either is waited on
  const uint64_t kraw = keys[(size_t)b * nk + min(lane, nk - 1)];
  const int sraw = SPARSE ? sel[(size_t)b * k + min(lane, k - 1)] : 0;
  if (wave == 0) {
    const uint64_t kv = wave_max_u64(lane < nk ? kraw : 0ull);
    if (lane == 0) *sh_M = key_value(kv);
    if (SPARSE && lane < k) sel_s[lane] = sraw;
  }
  if (SPARSE) {  // each slot's rank among the selected clusters (ascending cluster index)
    __syncthreads();
    if (tid < k) {
      const int sj = sel_s[tid];
      int r = 0;
#pragma unroll
      for (int j = 0; j < kMaxTopK; ++j) r += (j < k && sel_s[j] < sj) ? 1 : 0;
      rank2slot[r] = tid;
    }
  }
  __syncthreads();
}

// e of ordered elements r .. r + 3 (n % 4 == 0; zero past n) and their offset in the value array
template <bool SPARSE>
__device__ __forceinline__ size_t sample_load4(const float* vals, size_t rowbase, int n, int vsc, const int* rank2slot,
                                               int r, float M, float c, float* e) {
  const int rc = min(r, n - 4);
  size_t off = rowbase + rc;
  if (SPARSE) {
    const int seg = rc / vsc;  // vsc % 4 == 0: the 4 elements share a cluster
    off = rowbase + (size_t)rank2slot[seg] * vsc + (rc - seg * vsc);
  }
  const float4 v = *reinterpret_cast<const float4*>(vals + off);
  const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) e[i] = (r < n) ? exp2f((vv[i] - M) * c) : 0.f;
  return off;
}

// grid (tiles, B), kSampleThreads threads. vals: dense logits [B][n] or sparse logits [B][k][vsc] (n = k vsc).
template <bool SPARSE>
__global__ __launch_bounds__(kSampleThreads) void k_sample_tiles(int n, int vsc, int k, const float* vals,
                                                                 const int32_t* sel, const uint64_t* keys, int nk,
                                                                 float c, float* __restrict__ tsum) {
  __shared__ float sh_M;
  __shared__ int rank2slot[kMaxTopK];
  __shared__ float wpart[kSampleThreads / 64];
  const int t = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  sample_setup<SPARSE>(b, k, sel, keys, nk, &sh_M, rank2slot);
  float e[4];
  sample_load4<SPARSE>(vals, (size_t)b * n, n, vsc, rank2slot, t * kSampleTile + tid * 4, sh_M, c, e);
  const float s = wave_sum((e[0] + e[1]) + (e[2] + e[3]));
  if (lane_id() == 0) wpart[wave_id()] = s;
  __syncthreads();
  if (tid == 0) {
    float a = 0.f;
#pragma unroll
    for (int w = 0; w < kSampleThreads / 64; ++w) a += wpart[w];
    tsum[(size_t)b * kMaxSampleTiles + t] = a;
  }
}

// grid B, kSampleThreads threads. Writes the token and its probability to tok_out / prob_out[b * out_stride] and the
// token to tok_next[b] (each when set). ONE: the row's scored tokens fit one tile (the masked head); the total is
// then the block sum of the same e values and no tile sums are read.
template <bool SPARSE, bool ONE>
__global__ __launch_bounds__(kSampleThreads) void k_sample_pick(int n, int vsc, int k, const float* vals,
                                                                const int32_t* ids, const int32_t* sel,
                                                                const uint64_t* keys, int nk, float c,
                                                                const float* tsum, const float* u,
                                                                int32_t* tok_out, float* prob_out, int out_stride,
                                                                int32_t* tok_next) {
  __shared__ float sh_M, sh_P, sh_S, sh_target;
  __shared__ int sh_tile, sh_pick, sh_last;
  __shared__ int rank2slot[kMaxTopK];
  __shared__ float ts[kMaxSampleTiles];
  __shared__ float wtot[kSampleThreads / 64];
  const int b = blockIdx.x, tid = threadIdx.x, wave = wave_id(), lane = lane_id();
  const int ntiles = (n + kSampleTile - 1) / kSampleTile;
  const float ub = u[b];
  if (!ONE && tid < ntiles) ts[tid] = tsum[(size_t)b * kMaxSampleTiles + tid];
  if (tid == 0) {
    sh_pick = 0x7FFFFFFF;
    sh_last = -1;
  }
  sample_setup<SPARSE>(b, k, sel, keys, nk, &sh_M, rank2slot);
  if (ONE) {
    if (tid == 0) {
      sh_tile = 0;
      sh_P = 0.f;
    }
  } else if (tid == 0) {  // total, target, and the tile whose running sum first exceeds the target (in order)
    float S = 0.f;
    for (int t = 0; t < ntiles; ++t) S += ts[t];
    const float target = ub * S;
    float P = 0.f, Plast = 0.f;
    int tile = -1, last = 0;
    for (int t = 0; t < ntiles; ++t) {
      if (P + ts[t] > target) {
        tile = t;
        break;
      }
      if (ts[t] > 0.f) {
        last = t;
        Plast = P;
      }
      P += ts[t];
    }
    if (tile < 0) {  // rounding left the total at or below u * S: the last tile with mass (the row maximum has e = 1)
      tile = last;
      P = Plast;
    }
    sh_S = S;
    sh_P = P;
    sh_target = target;
    sh_tile = tile;
  }
  __syncthreads();
  const int r0 = sh_tile * kSampleTile + tid * 4;
  float e[4];
  const size_t off = sample_load4<SPARSE>(vals, (size_t)b * n, n, vsc, rank2slot, r0, sh_M, c, e);
  int4 idv = make_int4(0, 0, 0, 0);  // the four elements' token ids, fetched with their logits
  if (SPARSE) idv = *reinterpret_cast<const int4*>(ids + off);
  const float s = (e[0] + e[1]) + (e[2] + e[3]);
  // exclusive prefix of s over the block in thread order: wave inclusive scan, then the earlier waves' totals
  float incl = s;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float v = __shfl_up(incl, o, 64);
    if (lane >= o) incl += v;
  }
  if (lane == 63) wtot[wave] = incl;
  __syncthreads();
  float woff = 0.f;
  for (int w = 0; w < wave; ++w) woff += wtot[w];
  if (ONE) {  // every thread forms the same total from the wave totals
    float S = 0.f;
#pragma unroll
    for (int w = 0; w < kSampleThreads / 64; ++w) S += wtot[w];
    if (tid == 0) {
      sh_S = S;
      sh_target = ub * S;
    }
    __syncthreads();
  }
  float run = sh_P + woff + (incl - s);
  const float target = sh_target;
  int found = -1, lastpos = -1;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    run += e[i];
    if (found < 0 && run > target) found = i;
    if (e[i] > 0.f) lastpos = i;
  }
  if (found >= 0) atomicMin(&sh_pick, r0 + found);
  if (lastpos >= 0) atomicMax(&sh_last, r0 + lastpos);
  __syncthreads();
  const int pick = sh_pick != 0x7FFFFFFF ? sh_pick : sh_last;  // no crossing: rounding, take the last token with p > 0
  if (r0 <= pick && pick < r0 + 4) {
    const int i = pick - r0;
    const int iv[4] = {idv.x, idv.y, idv.z, idv.w};
    const int32_t token = SPARSE ? iv[i] : pick;
    const float prob = e[i] / sh_S;
    if (tok_out) tok_out[(size_t)b * out_stride] = token;
    if (prob_out) prob_out[(size_t)b * out_stride] = prob;
    if (tok_next) tok_next[b] = token;
  }
}

}  // namespace

// ------------------------------------------------------------------------------------------------------------
// launchers

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

hipError_t launch_topk_rows(hipStream_t s, int B, int C, int k, const float* scores, int32_t* sel) {
  if (k < 1 || k > kMaxTopK || k > C || C > kMaxCentroids) return hipErrorInvalidValue;
  const int npt = (C + 255) / 256;
  if (npt <= 2) return go(k_topk_rows<2>, B, 256, 0, s, C, k, scores, sel);
  if (npt <= 4) return go(k_topk_rows<4>, B, 256, 0, s, C, k, scores, sel);
  if (npt <= 8) return go(k_topk_rows<8>, B, 256, 0, s, C, k, scores, sel);
  return go(k_topk_rows<16>, B, 256, 0, s, C, k, scores, sel);
}

// the most (cluster, entry tile) pairs n selections of C clusters make: at most one partial tile per cluster
int group_tiles(int n, int C) { return (C < n ? C : n) + (n + kGroupTile - 1) / kGroupTile; }

hipError_t launch_group(hipStream_t s, int B, int C, int k, const int32_t* sel, int32_t* work) {
  const int n = B * k;
  if (n > kMaxBatch * kMaxTopK || C > kMaxCentroids) return hipErrorInvalidValue;
  const int T = group_tiles(n, C);
  return go(k_group, 1, 1024, 0, s, n, C, T, sel, reinterpret_cast<int4*>(work), work + 4 * T);
}

hipError_t launch_head_grouped(hipStream_t s, int B, int C, int k, int vsc, int H, const int32_t* ordering,
                               const uint16_t* Es, const float* h, const int32_t* work, int32_t* ids, float* z,
                               float* logits, size_t V, uint64_t* keys) {
  const int n = B * k;
  if (n > kMaxBatch * kMaxTopK || C > kMaxCentroids) return hipErrorInvalidValue;
  const int T = group_tiles(n, C);
  const int4* trec = reinterpret_cast<const int4*>(work);
  const int32_t* entries = work + 4 * T;
#define MTPD_HG(HCH_) \
  if (H == HCH_ * 128) \
    return go(k_head_grouped<HCH_>, T, 256, 0, s, k, vsc, ordering, Es, h, trec, entries, ids, z, logits, V, keys);
  MTPD_HG(2) MTPD_HG(4) MTPD_HG(6) MTPD_HG(8)
#undef MTPD_HG
  return hipErrorInvalidValue;
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

hipError_t launch_sample(hipStream_t s, int phase, int B, int n, int vsc, int k, const float* vals,
                         const int32_t* ids, const int32_t* sel, const uint64_t* keys, int nk, float temperature,
                         float* tsum, const float* u, int32_t* tok_out, float* prob_out, int out_stride,
                         int32_t* tok_next) {
  const int ntiles = (n + kSampleTile - 1) / kSampleTile;
  if (ntiles > kMaxSampleTiles || n % 4 != 0 || (k > 0 && vsc % 4 != 0)) return hipErrorInvalidValue;
  const float c = 1.4426950408889634f / temperature;
  if (phase == 0) {  // a single tile needs no tile sums: nothing to launch
    if (ntiles == 1) return hipSuccess;
    if (k > 0) return go(k_sample_tiles<true>, dim3(ntiles, B), kSampleThreads, 0, s, n, vsc, k, vals, sel, keys, nk, c, tsum);
    return go(k_sample_tiles<false>, dim3(ntiles, B), kSampleThreads, 0, s, n, vsc, k, vals, sel, keys, nk, c, tsum);
  }
#define MTPD_PICK(SP_, ONE_)                                                                                    \
  return go(k_sample_pick<SP_, ONE_>, B, kSampleThreads, 0, s, n, vsc, k, vals, ids, sel, keys, nk, c, tsum, u, \
            tok_out, prob_out, out_stride, tok_next)
  if (k > 0) {
    if (ntiles == 1) MTPD_PICK(true, true);
    MTPD_PICK(true, false);
  }
  if (ntiles == 1) MTPD_PICK(false, true);
  MTPD_PICK(false, false);
#undef MTPD_PICK
}

}  // namespace mtpd
