// Shared device/host helpers for the kvcc HIP library (gfx950, wave64).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "kvcc.h"

namespace kvcc {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int WAVE = 64;
constexpr double LOG2E_D = 1.4426950408889634;
constexpr float LN2_F = 0.69314718055994531f;

// Host-side helpers --------------------------------------------------------

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline int launch_status() {
  return hipGetLastError() == hipSuccess ? KV_OK : KV_ERR_LAUNCH;
}

inline float default_scale(float scale, int d) {
  return scale > 0.f ? scale : (float)(1.0 / __builtin_sqrt((double)d));
}

inline int ceil_div(int a, int b) { return (a + b - 1) / b; }
inline int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Per-kernel timing (kv_timing_enable): while it is on for `name`,
// timing_events hands out a start/stop event pair for one launch, and
// timing_done files the pair under `name`.
bool timing_events(const char* name, hipEvent_t* start, hipEvent_t* stop);
void timing_done(const char* name, hipEvent_t start, hipEvent_t stop, dim3 grid, dim3 block);

// kernel<<<grid, block, shmem, st>>>(args...).  While timing is on for
// `name`, the launch carries an event pair that the dispatch itself stamps at
// kernel start and end (hipExtLaunchKernelGGL), so timing adds no packets of
// its own to the stream.
template <typename K, typename... A>
inline void launch(const char* name, K kernel, dim3 grid, dim3 block, uint32_t shmem,
                   hipStream_t st, A... args) {
  hipEvent_t e0, e1;
  if (timing_events(name, &e0, &e1)) {
    hipExtLaunchKernelGGL(kernel, grid, block, shmem, st, e0, e1, 0, args...);
    timing_done(name, e0, e1, grid, block);
  } else {
    hipLaunchKernelGGL(kernel, grid, block, shmem, st, args...);
  }
}

// Device-side helpers ------------------------------------------------------

// 16-byte vector load/store through plain global accesses.
__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void st16(void* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Order-preserving uint32 key of an fp32 score (a larger score gives a
// larger key; -0.0 maps onto +0.0), and its inverse.  Selection ranks these
// keys; the score kernels histogram their top bits for it.
__device__ __forceinline__ uint32_t to_key(float s) {
  uint32_t u = __float_as_uint(s);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float from_key(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}
// The same key for the scores the score kernels write, in one instruction:
// those scores are sums of exponentials (+0.0 or positive, never -0.0 or
// negative), and for these to_key only sets the top bit.  The score pass's
// key histogram and the selection that reads it both use this mapping, so
// the two agree on any value the pass can write.
__device__ __forceinline__ uint32_t score_key(float s) {
  return __float_as_uint(s) | 0x80000000u;
}
// Bins of the top-digit key histogram (its top KEY_DIGIT bits).
constexpr int KEY_DIGIT = 11;
constexpr int KEY_BINS = 1 << KEY_DIGIT;

// exp2 / log2 on the hardware transcendental unit (v_exp_f32 / v_log_f32).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Wave-wide reductions (64 lanes).
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, WAVE));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, WAVE);
  return v;
}

// Inclusive prefix sum over the 64 lanes of a wave.
template <typename I>
__device__ __forceinline__ I wave_incl_scan(I v) {
  const int lane = threadIdx.x & (WAVE - 1);
#pragma unroll
  for (int o = 1; o < WAVE; o <<= 1) {
    I u = __shfl_up(v, o, WAVE);
    if (lane >= o) v += u;
  }
  return v;
}

// Set lanes of a wave-wide mask below the calling lane (v_mbcnt).
__device__ __forceinline__ uint32_t mbcnt(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Inclusive scans over a wave's 64 lanes with DPP moves: shifts by 1, 2, 4
// and 8 inside each 16-lane row, then lane 15 broadcast into rows 1 and 3
// and lane 31 into rows 2 and 3.  Lanes a move cannot source keep `id`.
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp_mov(uint32_t id, uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, CTRL, ROWS, 0xf, false);
}
template <class Op>
__device__ __forceinline__ uint32_t wave_scan_u32(uint32_t x, uint32_t id, Op op) {
  x = op(x, dpp_mov<0x111, 0xf>(id, x));
  x = op(x, dpp_mov<0x112, 0xf>(id, x));
  x = op(x, dpp_mov<0x114, 0xf>(id, x));
  x = op(x, dpp_mov<0x118, 0xf>(id, x));
  x = op(x, dpp_mov<0x142, 0xa>(id, x));
  x = op(x, dpp_mov<0x143, 0xc>(id, x));
  return x;
}
template <int CTRL, int ROWS>
__device__ __forceinline__ uint64_t dpp_add_step(uint64_t x) {
  const uint32_t lo = dpp_mov<CTRL, ROWS>(0u, (uint32_t)x);
  const uint32_t hi = dpp_mov<CTRL, ROWS>(0u, (uint32_t)(x >> 32));
  return x + (((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ uint64_t wave_scan_add_u64(uint64_t x) {
  x = dpp_add_step<0x111, 0xf>(x);
  x = dpp_add_step<0x112, 0xf>(x);
  x = dpp_add_step<0x114, 0xf>(x);
  x = dpp_add_step<0x118, 0xf>(x);
  x = dpp_add_step<0x142, 0xa>(x);
  x = dpp_add_step<0x143, 0xc>(x);
  return x;
}
struct OpAdd { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a + b; } };
struct OpMin { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a < b ? a : b; } };
struct OpMax { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a > b ? a : b; } };

// Sum over aligned groups of L lanes (L = 2, 4, ..., 32), result in every
// lane of the group.  DPP moves on the VALU: quad_perm swaps lanes 1 and 2
// apart, then the half-row mirror (lane i <-> 7-i) joins the two quads of an
// 8-lane group and the row mirror (i <-> 15-i) the two halves of a 16-lane
// row; 32-lane groups add the other row with one cross-row swizzle.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
template <int L>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(L >= 2 && L <= 32 && (L & (L - 1)) == 0, "group of 2..32 lanes");
  x += dpp_f32<0xB1>(x);                       // quad_perm [1,0,3,2]
  if constexpr (L >= 4) x += dpp_f32<0x4E>(x);  // quad_perm [2,3,0,1]
  if constexpr (L >= 8) x += dpp_f32<0x141>(x); // row_half_mirror
  if constexpr (L >= 16) x += dpp_f32<0x140>(x); // row_mirror
  if constexpr (L >= 32) x += __shfl_xor(x, 16, WAVE);
  return x;
}

// Value of lane 63 (the total of an inclusive scan), wave-uniform.
__device__ __forceinline__ uint32_t last_lane(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, WAVE - 1);
}
__device__ __forceinline__ uint64_t last_lane(uint64_t v) {
  return ((uint64_t)last_lane((uint32_t)(v >> 32)) << 32) | last_lane((uint32_t)v);
}

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int lane = threadIdx.x & (WAVE - 1);
  return lane == 0 ? 0ull : (~0ull >> (WAVE - lane));
}

}  // namespace kvcc
