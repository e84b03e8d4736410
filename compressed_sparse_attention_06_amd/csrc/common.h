// Device helpers shared by the gfx950 kernels: bf16 storage, matrix-core
// operand types, wave reductions and the RoPE angle.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "csa.h"
#include "rope_math.h"

namespace csa {

constexpr int kWave = 64;  // CDNA wavefront width

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float floatx4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float floatx16;

// ---------------------------------------------------------------------------
// bfloat16 storage (raw 16-bit patterns in memory)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// float -> bf16 bits, round to nearest even (inputs are finite)
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// Element i of a tensor of either dtype, as float.
__device__ __forceinline__ float load_elem(const void* p, int dtype, int64_t i) {
  if (dtype == CSA_BF16) return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
  return static_cast<const float*>(p)[i];
}
__device__ __forceinline__ void store_elem(void* p, int dtype, int64_t i, float v) {
  if (dtype == CSA_BF16)
    static_cast<uint16_t*>(p)[i] = static_cast<uint16_t>(f32_to_bf16_bits(v));
  else
    static_cast<float*>(p)[i] = v;
}

// 8 consecutive bf16 (16 bytes) as a matrix-core operand.
__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) {
  bf16x8 r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}

// ---------------------------------------------------------------------------
// Wave reductions and scans (64 lanes), register to register.  Within each
// 16-lane row, DPP lane moves: the two quad swaps (lane ^ 1, lane ^ 2), then
// the half-row mirror (lane 7 - i: the other quad of the half row) and the
// row mirror (lane 15 - i: the other half row), after which every lane of a
// row holds the row's result; the four rows then meet through the permlane
// swaps (lanes l ^ 32, then l ^ 16).
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_move(uint32_t x) {
  return uint32_t(__builtin_amdgcn_mov_dpp(int(x), CTRL, 0xF, 0xF, false));
}
template <typename Op>
__device__ __forceinline__ uint32_t wave_reduce_bits(uint32_t x, Op op) {
  x = op(x, dpp_move<0xB1>(x));   // quad_perm [1,0,3,2]
  x = op(x, dpp_move<0x4E>(x));   // quad_perm [2,3,0,1]
  x = op(x, dpp_move<0x141>(x));  // row_half_mirror
  x = op(x, dpp_move<0x140>(x));  // row_mirror
  const auto p = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  x = op(p[0], p[1]);
  const auto q = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  return op(q[0], q[1]);
}
__device__ __forceinline__ float wave_sum(float v) {
  return __uint_as_float(wave_reduce_bits(__float_as_uint(v), [](uint32_t a, uint32_t b) {
    return __float_as_uint(__uint_as_float(a) + __uint_as_float(b));
  }));
}
__device__ __forceinline__ float wave_max(float v) {
  return __uint_as_float(wave_reduce_bits(__float_as_uint(v), [](uint32_t a, uint32_t b) {
    return __float_as_uint(fmaxf(__uint_as_float(a), __uint_as_float(b)));
  }));
}
__device__ __forceinline__ float wave_min(float v) {
  return __uint_as_float(wave_reduce_bits(__float_as_uint(v), [](uint32_t a, uint32_t b) {
    return __float_as_uint(fminf(__uint_as_float(a), __uint_as_float(b)));
  }));
}
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
  return wave_reduce_bits(v, [](uint32_t a, uint32_t b) { return a + b; });
}
// Inclusive prefix sum over the wave's lanes: row_shr 1, 2, 4, 8 within each
// row (lanes shifted in from outside the row add 0), then every row adds the
// totals of the rows below it (lanes 15, 31, 47).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  x += uint32_t(__builtin_amdgcn_update_dpp(0, int(x), 0x111, 0xF, 0xF, false));
  x += uint32_t(__builtin_amdgcn_update_dpp(0, int(x), 0x112, 0xF, 0xF, false));
  x += uint32_t(__builtin_amdgcn_update_dpp(0, int(x), 0x114, 0xF, 0xF, false));
  x += uint32_t(__builtin_amdgcn_update_dpp(0, int(x), 0x118, 0xF, 0xF, false));
  const uint32_t r0 = __builtin_amdgcn_readlane(x, 15), r1 = __builtin_amdgcn_readlane(x, 31),
                 r2 = __builtin_amdgcn_readlane(x, 47);
  const int row = int(threadIdx.x % kWave) >> 4;
  return x + (row >= 1 ? r0 : 0u) + (row >= 2 ? r1 : 0u) + (row >= 3 ? r2 : 0u);
}

// ---------------------------------------------------------------------------
// RoPE rotation of pair i at position p (angle formed and reduced in double,
// see rope_math.h); the reduced angle goes through a single-precision sincos.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void rope_cos_sin(int64_t p, int i, int rope_dim, double log2_base,
                                             float* c, float* s) {
  sincosf(float(rope_angle(p, i, rope_dim, log2_base)), s, c);
}

constexpr float kLog2e = 1.4426950408889634f;

// 2^x on the hardware exponential (v_exp_f32).  Softmax arguments here are
// <= 0; results below 2^-126 flush to zero, which is harmless for weights.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Sum / max over the four 16-lane rows of a wave that share lane index
// l % 16 (lanes l, l^16, l^32, l^48), register to register: each swap
// exchanges one half of two copies of x, so adding (or max-ing) the pair
// combines lanes l and l^32, then l and l^16.
__device__ __forceinline__ float sum_rows4(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}
__device__ __forceinline__ float max_rows4(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
  const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
}

// max(x, 0) as one integer max on the bit pattern: a set sign bit makes the
// pattern a negative integer, so every negative value (and -0) becomes +0 and
// every other value passes unchanged.  fmaxf would add a NaN-quieting max.
__device__ __forceinline__ float relu(float x) {
  return __int_as_float(max(__float_as_int(x), 0));
}

}  // namespace csa
