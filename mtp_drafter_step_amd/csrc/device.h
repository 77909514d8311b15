// Device-side building blocks shared by the drafter-step kernels (gfx950, CDNA4, wave64): bf16 and key
// encodings, cross-lane reductions, and the launch helper that attaches timing events.
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
#ifndef MTPD_DEVICE_H
#define MTPD_DEVICE_H

#include "kernels.h"

#include <hip/hip_ext.h>

#include <math.h>
#include <stdlib.h>

#include <type_traits>

namespace mtpd {

// Timing events for the next launch only (see set_next_launch_events); defined in k_layers.hip.
extern thread_local hipEvent_t t_ev_start, t_ev_stop;

namespace {


constexpr int kRG = kRowGroup;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }
__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// fp32 -> bf16, round to nearest even (finite inputs)
// fp32 -> bf16, round to nearest even (the hardware conversion, v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
// two fp32 -> packed bf16 pair (a in the low half), one v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t f2bf2(float a, float b) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}
// the pair (a, b) as bf16 hi + lo parts (a + b within 2^-16 relative of hi + lo), each packed as by f2bf2
__device__ __forceinline__ void split_bf16x2(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = f2bf2(a, b);
  lo = f2bf2(a - bf_lo(hi), b - bf_hi(hi));
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
// the value of a (value, id) key (inverse of f32_order)
__device__ __forceinline__ float key_value(uint64_t k) {
  const uint32_t o = (uint32_t)(k >> 32);
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}
__device__ __forceinline__ int32_t key_id(uint64_t k) { return (int32_t)(0xFFFFFFFFu - (uint32_t)(k & 0xFFFFFFFFull)); }

__device__ __forceinline__ uint64_t u64_max(uint64_t a, uint64_t b) { return a > b ? a : b; }

// 16-byte load through the global address space: a generic (flat) load would also count against the LDS wait
// counter, so a wait for LDS reads would drain the outstanding memory loads too
__device__ __forceinline__ uint4 ld_global16(const void* p) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  return __builtin_bit_cast(uint4, *(const __attribute__((address_space(1))) u32x4*)(p));
}

// Transposing LDS read (ds_read_b64_tr_b16). Each lane names 4 consecutive 16-bit values (an 8-byte aligned LDS
// address); within each group of 16 lanes, take the 64 values the group names in lane order, and lane i of the group
// receives values i, 16 + i, 32 + i and 48 + i of that list. So when lane j of a group names row R + j / 4, columns
// C + 4 (j % 4) .. +4 of a row-major tile, lane i receives column C + i of rows R .. R + 3: a 4 x 16 block read
// column-wise, the B operand layout of a 16-deep matrix-core step. (Mapping established on gfx950 by reading an
// index-filled tile.)
__device__ __forceinline__ i16x4 lds_read_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(__attribute__((address_space(3))) void*)(p));
}

// GELU, tanh form: 0.5 a (1 + tanh(u)) with u = sqrt(2/pi) (a + 0.044715 a^3), evaluated as the equal a / (1 + e^-2u)
// on the hardware 2^x and reciprocal (a few ulp at every a; no cancellation in 1 + tanh(u) for negative a)
__device__ __forceinline__ float gelu_tanh(float a) {
  const float c = 0.7978845608028654f;  // sqrt(2/pi)
  const float u = c * (a + 0.044715f * a * a * a);
  return a * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-2.8853900817779268f * u));  // 2 log2(e)
}

// 1 / sqrt(x) on the hardware instruction (1 ulp): the RMSNorm scale, x >= eps > 0
__device__ __forceinline__ float rsqrt_hw(float x) { return __builtin_amdgcn_rsqf(x); }

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

// Maximum over the wave, left in every lane: the partners of XR's steps (lanes 32 and 16 apart, then within rows of
// 16 a rotation by 8, the half-row mirror and two quad permutations), all in the vector ALU; the halves of each
// 64-bit value move as exact bit patterns.
template <int O>
__device__ __forceinline__ uint32_t xr_partner_u32(uint32_t v) {
  return __float_as_uint(xr_partner<O>(__uint_as_float(v)));
}
template <int O>
__device__ __forceinline__ void max_step_u64(uint32_t& lo, uint32_t& hi) {
  const uint32_t plo = xr_partner_u32<O>(lo), phi = xr_partner_u32<O>(hi);
  const bool take = phi > hi || (phi == hi && plo > lo);
  lo = take ? plo : lo;
  hi = take ? phi : hi;
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
  max_step_u64<32>(lo, hi);
  max_step_u64<16>(lo, hi);
  max_step_u64<8>(lo, hi);
  max_step_u64<4>(lo, hi);
  max_step_u64<2>(lo, hi);
  max_step_u64<1>(lo, hi);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, xr_partner<32>(v));
  v = fmaxf(v, xr_partner<16>(v));
  v = fmaxf(v, xr_partner<8>(v));
  v = fmaxf(v, xr_partner<4>(v));
  v = fmaxf(v, xr_partner<2>(v));
  return fmaxf(v, xr_partner<1>(v));
}
// The value of the even (ODD = 0) or odd (ODD = 1) lane of each lane pair, by a quad permutation.
template <int ODD>
__device__ __forceinline__ uint32_t pair_lane(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, ODD ? 0xF5 : 0xA0, 0xf, 0xf, false);  // [1,1,3,3] / [0,0,2,2]
}

// a.lo * b.lo + a.hi * b.hi + c for two packed bf16 pairs, on the packed dot instruction (fp32 accumulation)
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
}

__device__ __forceinline__ void unpack4(uint2 w, float* f) {
  f[0] = bf_lo(w.x); f[1] = bf_hi(w.x); f[2] = bf_lo(w.y); f[3] = bf_hi(w.y);
}
__device__ __forceinline__ void unpack8(uint4 w, float* f) {
  f[0] = bf_lo(w.x); f[1] = bf_hi(w.x); f[2] = bf_lo(w.y); f[3] = bf_hi(w.y);
  f[4] = bf_lo(w.z); f[5] = bf_hi(w.z); f[6] = bf_lo(w.w); f[7] = bf_hi(w.w);
}

// Cache slot of key index t of a row's window: windows are given as [start, start + count) with start < cap and
// count <= cap, and indices past the end of the cache wrap to its beginning (ring-buffer caches)
__device__ __forceinline__ int slot_of(int t, int cap) { return t >= cap ? t - cap : t; }

inline int row_groups(int B) { return (B + kRG - 1) / kRG; }

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
}  // namespace mtpd

#endif  // MTPD_DEVICE_H
