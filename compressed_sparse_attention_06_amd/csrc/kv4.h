// Quantised compressed-KV rows: FP4 E2M1 latent, FP8 E4M3 RoPE tail.
//
// "Lab tổng hợp DeepSeek-V4.1-Flash", section "3 Giải pháp": the cache's
// per-token budget is priced with FP4 E2M1 for the latent and FP8 E4M3 for
// the rope tail; "LLM Atlas: DeepSeek", section "FP8 训练真正难在哪": low
// precision needs fine-grained scaling.  Layout of one row (D channels, the
// last rope_dim of them the tail, both multiples of 32):
//   [latent codes: (D-rope)/2 bytes, even channel in the low nibble]
//   [tail codes: rope bytes]
//   [scale bytes: one per 32 channels, latent blocks then tail blocks]
//   [zero padding to a multiple of 16 bytes]
// A block of 32 channels shares the scale 2^x (byte x + 127): the smallest x
// with max|v| / 2^x <= 6 (E2M1) or 448 (E4M3), so nothing clips.  Elements
// round to the nearest code, ties to the even code; a value rounding to zero
// keeps its sign.  D = 512 with a 64-wide tail: 304 bytes per row.
#pragma once

#include "common.h"

namespace csa {

constexpr int kKV4Block = 32;

__host__ __device__ inline int kv4_row_bytes(int D, int rope_dim) {
  const int lat = D - rope_dim;
  const int raw = lat / 2 + rope_dim + lat / kKV4Block + rope_dim / kKV4Block;
  return (raw + 15) / 16 * 16;
}

// Byte offsets, within a row, of the codes and of the scale of the 8
// channels ch .. ch+7 (ch a multiple of 8).
__host__ __device__ inline int kv4_code_offset(int ch, int D, int rope_dim) {
  const int lat = D - rope_dim;
  return ch < lat ? ch / 2 : lat / 2 + (ch - lat);
}
__host__ __device__ inline int kv4_scale_offset(int ch, int D, int rope_dim) {
  return (D - rope_dim) / 2 + rope_dim + ch / kKV4Block;
}

// Scale exponent of a block whose largest magnitude is amax (exact, from the
// fp32 bits: amax = (1 + f) 2^e; E2M1 takes x = e - 2 when 1 + f <= 1.5, else
// e - 1; E4M3 takes x = e - 8 when 1 + f <= 1.75, else e - 7), at least -127.
__device__ __forceinline__ int kv4_scale_exp(float amax, bool fp4) {
  if (!(amax > 0.f)) return -127;
  const uint32_t u = __float_as_uint(amax);
  const int e = int((u >> 23) & 0xffu) - 127;
  if (e == -127) return -127;  // a subnormal maximum: every choice lies below -127
  const uint32_t m = u & 0x7fffffu;
  const int x = fp4 ? (m <= 0x400000u ? e - 2 : e - 1) : (m <= 0x600000u ? e - 8 : e - 7);
  return x < -127 ? -127 : x;
}

// E2M1 code of y (|y| <= 6): the magnitude code counts the midpoints passed,
// a tie staying on the even code.
__device__ __forceinline__ uint32_t e2m1_code(float y) {
  const float a = fabsf(y);
  const uint32_t mag = uint32_t(a > 0.25f) + uint32_t(a >= 0.75f) + uint32_t(a > 1.25f) + uint32_t(a >= 1.75f) +
                       uint32_t(a > 2.5f) + uint32_t(a >= 3.5f) + uint32_t(a > 5.f);
  return ((__float_as_uint(y) >> 28) & 8u) | mag;
}

// E4M3 code of y (|y| <= 448): round to nearest even on the fp32 bits;
// below 2^-6 the code counts units of 2^-9.
__device__ __forceinline__ uint32_t e4m3_code(float y) {
  const uint32_t s = (__float_as_uint(y) >> 24) & 0x80u;
  const float a = fabsf(y);
  if (a < 0.015625f) return s | uint32_t(__builtin_rintf(a * 512.f));  // rint: ties to even; 8 = 2^-6
  const uint32_t u = __float_as_uint(a);
  int e = int((u >> 23) & 0xffu) - 127;
  uint32_t r = (u >> 20) & 7u;
  const uint32_t rem = u & 0xfffffu;
  if (rem > 0x80000u || (rem == 0x80000u && (r & 1u))) ++r;
  if (r == 8u) {
    r = 0;
    ++e;
  }
  return s | (uint32_t(e + 7) << 3) | r;
}

__device__ __forceinline__ float e2m1_value(uint32_t c) {
  const uint32_t e = (c >> 1) & 3u, m = c & 1u;
  const uint32_t mag = e == 0 ? (m ? 0x3F000000u : 0u) : (((e + 126u) << 23) | (m << 22));
  return __uint_as_float(mag | ((c & 8u) << 28));
}

__device__ __forceinline__ float e4m3_value(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  const float mag = e == 0 ? float(m) * (1.f / 512.f) : __uint_as_float(((e + 120u) << 23) | (m << 20));
  return __uint_as_float(__float_as_uint(mag) | ((c & 0x80u) << 24));
}

// The 8 channels of one lane as bf16 (exact: the codes carry at most 4
// significant bits and the scale is a power of two): `codes` holds the lane's
// code bytes (4 for E2M1 in .x, 8 for E4M3), `sbyte` its block's scale byte.
// gfx950's scaled pair conversions (FP4 pair from one byte, FP8 pair from one
// 16-bit half; the even channel lands in the low half) do the decoding; they
// agree bit for bit with e2m1_value / e4m3_value times the scale on every
// code.
__device__ __forceinline__ uint4 kv4_lane_bf16(uint2 codes, uint32_t sbyte, bool fp4) {
  const float sc = __builtin_ldexpf(1.f, int(sbyte & 0xffu) - 127);
  uint32_t w[4];
  auto bits = [](auto v) {
    uint32_t u;
    __builtin_memcpy(&u, &v, 4);
    return u;
  };
  if (fp4) {
    w[0] = bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes.x, sc, 0));
    w[1] = bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes.x, sc, 1));
    w[2] = bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes.x, sc, 2));
    w[3] = bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes.x, sc, 3));
  } else {
    w[0] = bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes.x, sc, false));
    w[1] = bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes.x, sc, true));
    w[2] = bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes.y, sc, false));
    w[3] = bits(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes.y, sc, true));
  }
  return uint4{w[0], w[1], w[2], w[3]};
}

// Channel d of a quantised row, as float.
__device__ __forceinline__ float kv4_elem(const unsigned char* row, int d, int D, int rope_dim) {
  const int lat = D - rope_dim;
  const int x = int(row[kv4_scale_offset(d, D, rope_dim)]) - 127;
  float v;
  if (d < lat) {
    const uint32_t byte = row[d / 2];
    v = e2m1_value((d & 1) ? (byte >> 4) : (byte & 15u));
  } else {
    v = e4m3_value(row[lat / 2 + (d - lat)]);
  }
  return __builtin_ldexpf(v, x);
}

// One wave writes the quantised row of D fp32 values y (LDS or registers
// read through the pointer).  Lane l takes channels 512c + 8l .. +7 of chunk
// c; the four lanes of a 32-channel block meet through DPP quad moves.
__device__ __forceinline__ void kv4_store_row(const float* y, int D, int rope_dim, unsigned char* row) {
  const int lane = threadIdx.x % kWave;
  const int lat = D - rope_dim;
  for (int c0 = 0; c0 < D; c0 += 8 * kWave) {
    const int ch = c0 + 8 * lane;
    const bool in = ch < D;
    float v[8];
    float am = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[i] = in ? y[ch + i] : 0.f;
      am = fmaxf(am, fabsf(v[i]));
    }
    // the block's largest magnitude: max over the lane quad
    am = fmaxf(am, __uint_as_float(dpp_move<0xB1>(__float_as_uint(am))));
    am = fmaxf(am, __uint_as_float(dpp_move<0x4E>(__float_as_uint(am))));
    if (!in) continue;
    const bool fp4 = ch < lat;
    const int x = kv4_scale_exp(am, fp4);
    if (fp4) {
      uint32_t w = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) w |= e2m1_code(__builtin_ldexpf(v[i], -x)) << (4 * i);
      *reinterpret_cast<uint32_t*>(row + ch / 2) = w;
    } else {
      uint32_t w0 = 0, w1 = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        w0 |= e4m3_code(__builtin_ldexpf(v[i], -x)) << (8 * i);
        w1 |= e4m3_code(__builtin_ldexpf(v[4 + i], -x)) << (8 * i);
      }
      *reinterpret_cast<uint2*>(row + lat / 2 + (ch - lat)) = uint2{w0, w1};
    }
    if (lane % 4 == 0) row[kv4_scale_offset(ch, D, rope_dim)] = static_cast<unsigned char>(x + 127);
  }
  // zero padding after the scale bytes
  const int raw = lat / 2 + rope_dim + D / kKV4Block;
  for (int p = raw + lane; p < kv4_row_bytes(D, rope_dim); p += kWave) row[p] = 0;
}

}  // namespace csa
