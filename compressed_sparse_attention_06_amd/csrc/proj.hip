// Projections on either side of the attention: the low-rank query path and
// the grouped output projection.
//
// "DeepSeek-V4-Flash 架构：一个 token 的旅程", section "低秩 Q：两次矩阵乘法接起来"
// (down-projection of the hidden state to a 1024-wide latent, RMSNorm,
// up-projection to 64 heads of 512, per-head RMS normalisation, RoPE on the
// last 64 dims) and section "输出投影也分组，并且降低中间维度" (8 groups of 8
// heads, one 1024x4096 down-projection per group, then one 4096x8192 matrix
// back to the model width).
//
// At decode the token count M is small and each projection streams its
// weight matrix from HBM once: ~8 flop per weight byte at M = 8, far under
// the matrix cores' ridge, so the kernel is built to keep HBM busy.  A block
// owns 128 output rows (weight rows; a 16-row tile per wave), one K chunk
// and up to 32 tokens; the K chunks of one row tile run in different blocks
// (enough blocks to spread the weights over the chip) and leave fp32
// partials that the next step sums.  Each lane reads 64 contiguous bytes of
// a weight row per 128-wide K block (16 rows x 256 B per wave), which the
// matrix core consumes as four 16x16x32 bf16 products whose K chunks are
// permuted the same way on both operands.  Activations are tiny and
// L2-resident; an fp32 activation is split into a bf16 head and a bf16
// remainder (two products), so the contraction keeps ~16 mantissa bits of it.
#include "common.h"
#include "kernels.h"

namespace csa {
namespace {

constexpr int kPW = 8;                 // waves per block
constexpr int kPThreads = kPW * kWave;
constexpr int kKB = 128;               // K block: 4 MFMA steps of 32


// Matrix-core operand of 8 bf16 from LDS.
__device__ __forceinline__ bf16x8 lds_frag(const uint16_t* p) { return as_bf16x8(*reinterpret_cast<const uint4*>(p)); }

// C[g][m][n] = sum_k A[g][m][k] * W[g][n][k] over one K chunk of kc = 128*NKB.
// grid.x = row groups (128 rows, one 16-row tile per wave) x groups,
// grid.y = K chunks, grid.z = token chunks of 16*MT.  The block stages its
// token rows of the chunk in LDS once (an fp32 activation as a bf16 head and
// a bf16 remainder), while every wave has its whole weight tile of the chunk
// (16 rows x kc) in flight; the waves then run their products from
// registers and LDS.  One K chunk: C is written directly; several: fp32
// partials per chunk, summed (in chunk order) by whatever reads them next.
template <int MT, bool ACT_F32, int NKB>
__global__ __launch_bounds__(kPThreads) void proj_gemm(ProjArgs a) {
  constexpr int kc = NKB * kKB;
  constexpr int pitch = kc + 8;  // bf16 per LDS row: rows 16 bytes apart in the banks
  constexpr int rows = 16 * MT;
  __shared__ __attribute__((aligned(16))) uint16_t act[(ACT_F32 ? 2 : 1) * rows * pitch];  // hi rows, then lo
  const int lane = threadIdx.x % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int c16 = lane % 16, gq = lane / 16;
  const int rgroups = (a.N + 127) / 128;
  const int grp = int(blockIdx.x) / rgroups;
  const int n0 = (int(blockIdx.x) % rgroups) * 128 + wave * 16;
  const int ks = blockIdx.y;
  const int64_t k0 = int64_t(ks) * kc;
  const int m0 = int(blockIdx.z) * rows;
  const bool live = n0 < a.N;  // a wave past the last row still helps stage

  // 1. token rows of the chunk: loads first (weights queue behind them).
  // Every thread issues the same loads (rows past the last token read the
  // last token's row and are zeroed when staged): behind a per-thread branch
  // the compiler waited for each load before issuing the next, a chain of
  // round trips ahead of the weight stream.
  constexpr int per_thread = rows * kc / 4 / kPThreads;  // 4 values per slot
  static_assert(per_thread >= 1 && rows * kc / 4 % kPThreads == 0, "staging slots");
  constexpr int RW = ACT_F32 ? 4 : 2;  // 32-bit words per slot
  uint32_t xr[per_thread][RW];
  auto slot_off = [&](int i, bool* valid) {
    const int slot = i * kPThreads + int(threadIdx.x);
    const int r = slot / (kc / 4), c = (slot % (kc / 4)) * 4;
    const int m = m0 + r;
    *valid = m < a.M;
    return int64_t(grp) * a.a_goff + int64_t(m < a.M ? m : a.M - 1) * a.lda + k0 + c;
  };
#pragma unroll
  for (int i = 0; i < per_thread; ++i) {
    bool valid;
    const int64_t off = slot_off(i, &valid);
    if constexpr (ACT_F32) {
      const uint4 v = *reinterpret_cast<const uint4*>(static_cast<const float*>(a.A) + off);
      xr[i][0] = v.x; xr[i][1] = v.y; xr[i][2] = v.z; xr[i][3] = v.w;
    } else {
      const uint2 u = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(a.A) + off);
      xr[i][0] = u.x; xr[i][1] = u.y;
    }
  }
  __builtin_amdgcn_sched_barrier(0);  // (keeps the token rows' loads ahead of the weights')
  // 2. the wave's whole weight tile of the chunk: 64 contiguous bytes of one
  // row per lane and K block (issued by every wave: rows past the last read
  // the last row, and their products are not stored)
  uint4 w[NKB][4];
  {
    const int nrow = n0 + c16 < a.N ? n0 + c16 : a.N - 1;
    const uint4* W = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.W) + int64_t(grp) * a.w_goff +
                                                    int64_t(nrow) * a.K + k0 + 32 * gq);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int s = 0; s < 4; ++s) w[kb][s] = W[kb * (kKB / 8) + s];  // plain loads: measured faster than non-temporal
  }
  // 3. fp32 rows that are partial sums of the previous product add their
  // other parts, in order: one batch of loads per part, every slot at once
  // (those loads queue behind the weights)
  float v[per_thread][4];
  if constexpr (ACT_F32) {
#pragma unroll
    for (int i = 0; i < per_thread; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) v[i][j] = __uint_as_float(xr[i][j]);
    for (int p = 1; p < a.a_nsum; ++p) {
      float4 u[per_thread];
#pragma unroll
      for (int i = 0; i < per_thread; ++i) {
        bool valid;
        const int64_t off = slot_off(i, &valid);
        u[i] = *reinterpret_cast<const float4*>(static_cast<const float*>(a.A) + off + p * a.a_kstride);
      }
#pragma unroll
      for (int i = 0; i < per_thread; ++i) {
        v[i][0] += u[i].x; v[i][1] += u[i].y; v[i][2] += u[i].z; v[i][3] += u[i].w;
      }
    }
  }
  // 4. stage the token rows (bf16, or a bf16 head and remainder)
#pragma unroll
  for (int i = 0; i < per_thread; ++i) {
    bool valid;
    (void)slot_off(i, &valid);
    const int slot = i * kPThreads + int(threadIdx.x);
    const int r = slot / (kc / 4), c = (slot % (kc / 4)) * 4;
    if constexpr (ACT_F32) {
#pragma unroll
      for (int j = 0; j < 4; ++j) v[i][j] = valid ? v[i][j] : 0.f;
      const uint32_t h0 = f32_to_bf16_bits(v[i][0]), h1 = f32_to_bf16_bits(v[i][1]);
      const uint32_t h2 = f32_to_bf16_bits(v[i][2]), h3 = f32_to_bf16_bits(v[i][3]);
      *reinterpret_cast<uint2*>(&act[r * pitch + c]) = uint2{h0 | (h1 << 16), h2 | (h3 << 16)};
      const uint32_t l0 = f32_to_bf16_bits(v[i][0] - __uint_as_float(h0 << 16));
      const uint32_t l1 = f32_to_bf16_bits(v[i][1] - __uint_as_float(h1 << 16));
      const uint32_t l2 = f32_to_bf16_bits(v[i][2] - __uint_as_float(h2 << 16));
      const uint32_t l3 = f32_to_bf16_bits(v[i][3] - __uint_as_float(h3 << 16));
      *reinterpret_cast<uint2*>(&act[rows * pitch + r * pitch + c]) = uint2{l0 | (l1 << 16), l2 | (l3 << 16)};
    } else {
      // bf16 rows go to LDS as they are
      *reinterpret_cast<uint2*>(&act[r * pitch + c]) = valid ? uint2{xr[i][0], xr[i][1]} : uint2{0u, 0u};
    }
  }
  __syncthreads();
  if (!live) return;
  // 5. products: K chunk j of 8 (j = 4*gq + s within a K block) pairs the
  // lane's weight bytes with the same 8 K values of token row c16
  floatx4 acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const bf16x8 wf = as_bf16x8(w[kb][s]);
      const int kk = kb * kKB + 32 * gq + 8 * s;
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const int r = t * 16 + c16;
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf, lds_frag(&act[r * pitch + kk]), acc[t], 0, 0, 0);
        if constexpr (ACT_F32)
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf, lds_frag(&act[(rows + r) * pitch + kk]), acc[t],
                                                            0, 0, 0);
      }
    }
  }
  // 6. lane (c16, gq) holds rows n0 + 4*gq + i of token m0 + 16*t + c16
  const bool partial = a.ks_count > 1;
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int m = m0 + t * 16 + c16;
    if (m >= a.M) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int n = n0 + 4 * gq + i;
      if (n >= a.N) continue;
      const int64_t o = int64_t(grp) * a.c_goff + int64_t(m) * a.ldc + n;
      if (partial) a.part[int64_t(ks) * a.part_kstride + o] = acc[t][i];
      else store_elem(a.C, a.c_dtype, o, acc[t][i]);
    }
  }
}

// C = sum over ks of part[ks] (fp32, in chunk order): grid (M, ceil(N/256)).
__global__ __launch_bounds__(256) void proj_reduce(ProjArgs a) {
  const int m = blockIdx.x, n = int(blockIdx.y) * 256 + int(threadIdx.x);
  if (n >= a.N * a.groups) return;
  const int grp = n / a.N, nn = n % a.N;
  const int64_t o = int64_t(grp) * a.c_goff + int64_t(m) * a.ldc + nn;
  float v = a.part[o];
  for (int k = 1; k < a.ks_count; ++k) v += a.part[int64_t(k) * a.part_kstride + o];
  store_elem(a.C, a.c_dtype, o, v);
}

// Row normalisation with optional gain and RoPE: for token m and column
// group j (cols [j*G, (j+1)*G)), y = x / sqrt(mean(x^2) + eps) * gamma, then
// the trailing rope_dim columns of the group turn by position pos[m].
// grid (M, ncols / G), up to 1024 threads (one column each when G allows).
__global__ __launch_bounds__(1024) void rows_norm(NormArgs a) {
  extern __shared__ float xs[];  // G values, then 16 wave sums
  const int m = blockIdx.x, j = blockIdx.y;
  const float* x = a.x + int64_t(m) * a.ldx + int64_t(j) * a.G;
  float ss = 0.f;
  for (int c = threadIdx.x; c < a.G; c += blockDim.x) {
    // the K-chunk partials of the product that made x, added in chunk order;
    // eight loads go out before the first add
    float v = 0.f;
    int p = 0;
    for (; p + 8 <= a.x_nsum; p += 8) {
      float u[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) u[i] = x[c + (p + i) * a.x_kstride];
#pragma unroll
      for (int i = 0; i < 8; ++i) v += u[i];
    }
    for (; p < a.x_nsum; ++p) v += x[c + p * a.x_kstride];
    xs[c] = v;
    ss = fmaf(v, v, ss);
  }
  float* red = xs + a.G;
  ss = wave_sum(ss);
  if (threadIdx.x % kWave == 0) red[threadIdx.x / kWave] = ss;
  __syncthreads();
  float tot = 0.f;
  for (int w = 0; w < int(blockDim.x) / kWave; ++w) tot += red[w];
  const float inv = rsqrtf(tot / float(a.G) + a.eps);
  const int r0 = a.G - a.rope_dim;
  const int64_t p = a.pos ? a.pos[m] : 0;
  const int64_t yo = int64_t(m) * a.ldy + int64_t(j) * a.G;
  for (int c = threadIdx.x; c < a.G; c += blockDim.x) {
    if (c >= r0 && ((c - r0) & 1)) continue;  // odd rope channels go with their even partner
    const float g0 = a.gamma ? a.gamma[c] : 1.f;
    const float y0 = xs[c] * inv * g0;
    if (c < r0) {
      store_elem(a.y, a.y_dtype, yo + c, y0);
    } else {
      const float g1 = a.gamma ? a.gamma[c + 1] : 1.f;
      const float y1 = xs[c + 1] * inv * g1;
      float cs, sn;
      rope_cos_sin(p, (c - r0) / 2, a.rope_dim, a.rope_log2_base, &cs, &sn);
      store_elem(a.y, a.y_dtype, yo + c, y0 * cs - y1 * sn);
      store_elem(a.y, a.y_dtype, yo + c + 1, y0 * sn + y1 * cs);
    }
  }
}

}  // namespace

ProjPlan plan_proj(int M, int N, int K, int groups, bool act_f32) {
  ProjPlan p{};
  p.mt = M <= 16 ? 1 : 2;
  const int mchunks = (M + 16 * p.mt - 1) / (16 * p.mt);
  const int kc_max = (p.mt == 2 && act_f32) ? 512 : 1024;
  const int64_t rg = int64_t((N + 127) / 128) * groups;
  // the largest chunk that still spreads the weights over the chip (about
  // one block per compute unit), at least two K blocks per wave when K allows
  int kc = 0;
  for (int c = kc_max; c >= 256; c /= 2) {
    if (K % c != 0) continue;
    kc = c;
    if (rg * (K / c) * mchunks >= 256) break;
  }
  if (kc == 0) kc = 128;
  p.kc = kc;
  p.ks = K / kc;
  p.mchunks = mchunks;
  return p;
}

hipError_t launch_proj_gemm(const ProjArgs& a, hipStream_t stream) {
  if (a.M == 0 || a.N == 0) return hipSuccess;
  const ProjPlan p = plan_proj(a.M, a.N, a.K, a.groups, a.a_dtype == CSA_F32);
  if (p.kc != a.kc || p.ks != a.ks_count) return hipErrorInvalidValue;  // the caller planned another split
  const dim3 grid(unsigned((a.N + 127) / 128 * a.groups), unsigned(p.ks), unsigned(p.mchunks));
  const bool f32 = a.a_dtype == CSA_F32;
#define CSA_PROJ_CASE(MT, F, NKB)                                                                        \
  if (p.mt == MT && f32 == F && p.kc == NKB * kKB) {                                                     \
    hipLaunchKernelGGL((proj_gemm<MT, F, NKB>), grid, dim3(kPThreads), 0, stream, a);                    \
    return hipGetLastError();                                                                            \
  }
  CSA_PROJ_CASE(1, true, 8) CSA_PROJ_CASE(1, true, 4) CSA_PROJ_CASE(1, true, 2) CSA_PROJ_CASE(1, true, 1)
  CSA_PROJ_CASE(1, false, 8) CSA_PROJ_CASE(1, false, 4) CSA_PROJ_CASE(1, false, 2) CSA_PROJ_CASE(1, false, 1)
  CSA_PROJ_CASE(2, true, 4) CSA_PROJ_CASE(2, true, 2) CSA_PROJ_CASE(2, true, 1)
  CSA_PROJ_CASE(2, false, 8) CSA_PROJ_CASE(2, false, 4) CSA_PROJ_CASE(2, false, 2) CSA_PROJ_CASE(2, false, 1)
#undef CSA_PROJ_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_proj_reduce(const ProjArgs& a, hipStream_t stream) {
  if (a.M == 0 || a.N == 0) return hipSuccess;
  hipLaunchKernelGGL(proj_reduce, dim3(unsigned(a.M), unsigned((int64_t(a.N) * a.groups + 255) / 256)), dim3(256), 0,
                     stream, a);
  return hipGetLastError();
}

hipError_t launch_rows_norm(const NormArgs& a, int ngroups, hipStream_t stream) {
  if (a.M == 0 || ngroups == 0) return hipSuccess;
  const int threads = a.G >= 1024 ? 1024 : (a.G + kWave - 1) / kWave * kWave;
  hipLaunchKernelGGL(rows_norm, dim3(unsigned(a.M), unsigned(ngroups)), dim3(threads),
                     (size_t(a.G) + 16) * sizeof(float), stream, a);
  return hipGetLastError();
}

}  // namespace csa
