// Internal device helpers for libddtree (gfx950, wave64). Not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ddtree.h"
#include "launch.hpp"

namespace ddt {

constexpr int kWave = 64;

// Order-preserving map of a finite fp32 onto uint32: a < b  <=>  key(a) <
// key(b), with -0 and +0 mapped to the same key.
__device__ __forceinline__ uint32_t f32_key(float x) {
  uint32_t u = __float_as_uint(x);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_f32(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}

__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    uint32_t o = __shfl_xor(v, off, kWave);
    v = o > v ? o : v;
  }
  return v;
}

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// DPP-based reductions: a fixed butterfly inside each 16-lane row
// (quad xor 1, quad xor 2, half-row mirror, row mirror), then the four row
// results are read into scalar registers and combined in a fixed order.
// The result is wave-uniform and bit-reproducible.
constexpr int kDppQuadXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;  // lane i <-> 7 - i within 8 lanes
constexpr int kDppRowMirror = 0x140;      // lane i <-> 15 - i within 16 lanes

// Every pattern above reads a lane of the same row, so each lane gets a
// value: a plain DPP move (bound_ctrl), which needs no copy of an old value
// and can fuse into the consuming instruction.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}

struct OpMax {
  __device__ __forceinline__ float operator()(float a, float b) const { return fmaxf(a, b); }
};
struct OpMin {
  __device__ __forceinline__ float operator()(float a, float b) const { return fminf(a, b); }
};
struct OpSum {
  __device__ __forceinline__ float operator()(float a, float b) const { return a + b; }
};

template <class Op>
__device__ __forceinline__ float wave_reduce_uniform(float v, Op op) {
  v = op(v, dpp_f32<kDppQuadXor1>(v));
  v = op(v, dpp_f32<kDppQuadXor2>(v));
  v = op(v, dpp_f32<kDppRowHalfMirror>(v));
  v = op(v, dpp_f32<kDppRowMirror>(v));
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return op(op(a, b), op(c, d));
}

// Ballot across the wave as a 64-bit mask.
__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

// Number of set bits of `mask` below this lane.
__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

}  // namespace ddt
