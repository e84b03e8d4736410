// Indexer scoring: score[e] = sum_h w[h] * relu(q_idx[h] . idx_cache[e]).
//
// "DeepSeek-V4-Flash 架构：一个 token 的旅程", section "少读 KV 之前，Indexer
// 仍要给历史打分" (64 heads of dim 128 over one shared 128-d index cache,
// signed weights); "Lab tổng hợp DeepSeek-V4.1-Flash", section "3 Giải pháp"
// (ReLU on each head's dot product).
//
// Every 256-byte index row meets 64 heads x 128 dims: 64 flop per byte, more
// than a vector-ALU roofline can stream at HBM rate, so the 64 heads form the
// M side of a bf16 matrix-core product even for a single query.  Two kernels:
//
//  * index_stream (few queries, e.g. decode): each wave keeps the query's
//    64x128 operand in registers and streams 64 index rows per step straight
//    from HBM into registers (each lane reads 64 contiguous bytes of one row),
//    4 x 16x16x32 MFMA per 16 rows and K-step, then ReLU, head weights and a
//    two-step cross-lane sum.  Pure streaming: no LDS.
//  * index_tile (many queries, e.g. prefill): a workgroup keeps a tile of
//    index rows stationary in registers and streams query operands through
//    LDS; causal tiles that no query of the block can see are skipped.
//
// Both use the same K-order inside an MFMA K-step (lane group g, element i
// <-> dim g*32 + ks*8 + i) for A and B, which the contraction allows.
#include "common.h"
#include "kernels.h"

namespace csa {
namespace {

constexpr int kHI = 64;   // indexer heads on the matrix-core path
constexpr int kDI = 128;  // indexer head dim on the matrix-core path

__device__ __forceinline__ int64_t visible_entries(const int* pos, int64_t qi, int ratio, int Ncap) {
  const int p = pos[qi];
  const int64_t nv = p >= 0 ? (int64_t(p) + 1) / ratio : 0;
  return nv < Ncap ? nv : Ncap;
}

// ---------------------------------------------------------------------------
// Streaming kernel: grid (ceil(Ncap / 256), B*S), 4 waves x 64 entries.
// ---------------------------------------------------------------------------
constexpr int kStreamWaves = 4;
constexpr int kStreamRows = 64;  // rows per wave
constexpr int kStreamBlockRows = kStreamWaves * kStreamRows;

__global__ __launch_bounds__(kWave* kStreamWaves) void index_stream(IndexArgs a) {
  const int64_t qi = blockIdx.x;
  const int b = int(qi / a.S);
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int g = lane / 16, r16 = lane % 16;
  const int Ncap = a.Ncap;
  const int64_t n_vis = visible_entries(a.pos, qi, a.ratio, Ncap);
  const int64_t e_base = int64_t(blockIdx.y) * kStreamBlockRows + wave * kStreamRows;
  float* srow = a.scores + qi * Ncap;

  if (e_base >= n_vis) {  // nothing visible in this wave's rows
    const int64_t e = e_base + lane;
    if (e < Ncap) srow[e] = -INFINITY;
    return;
  }

  const uint16_t* q = static_cast<const uint16_t*>(a.q_idx) + qi * (kHI * kDI);
  bf16x8 qa[4][4];  // [head tile][K-step]
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      qa[mt][ks] = as_bf16x8(*reinterpret_cast<const uint4*>(q + (mt * 16 + r16) * kDI + g * 32 + ks * 8));
  float wv[4][4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) wv[mt][i] = a.w[qi * kHI + mt * 16 + g * 4 + i];

  const uint16_t* cache = static_cast<const uint16_t*>(a.cache) + int64_t(b) * Ncap * kDI;
  uint4 kb[4][4];  // [16-row block][K-step]
#pragma unroll
  for (int blk = 0; blk < 4; ++blk) {
    const int64_t e = e_base + blk * 16 + r16;
    if (e < n_vis) {
      const uint4* src = reinterpret_cast<const uint4*>(cache + e * kDI + g * 32);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) kb[blk][ks] = src[ks];
    } else {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) kb[blk][ks] = uint4{0, 0, 0, 0};
    }
  }
#pragma unroll
  for (int blk = 0; blk < 4; ++blk) {
    floatx4 acc[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) acc[mt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8 kk = as_bf16x8(kb[blk][ks]);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[mt][ks], kk, acc[mt], 0, 0, 0);
    }
    // lane holds heads mt*16 + g*4 + i of row r16
    float part = 0.f;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) part += fmaxf(acc[mt][i], 0.f) * wv[mt][i];
    part += __shfl_xor(part, 16, kWave);
    part += __shfl_xor(part, 32, kWave);
    const int64_t e = e_base + blk * 16 + r16;
    if (g == 0 && e < Ncap) srow[e] = e < n_vis ? part : -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// Vector-ALU kernel for other shapes / fp32: one thread per (query, entry).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void index_any(IndexArgs a) {
  extern __shared__ float qs[];  // H*D query values, then H weights
  const int64_t qi = blockIdx.x;
  const int b = int(qi / a.S);
  const int H = a.H, D = a.D;
  for (int i = threadIdx.x; i < H * D; i += blockDim.x)
    qs[i] = load_elem(a.q_idx, a.dtype, qi * H * D + i);
  for (int i = threadIdx.x; i < H; i += blockDim.x) qs[H * D + i] = a.w[qi * H + i];
  __syncthreads();
  const int64_t e = int64_t(blockIdx.y) * blockDim.x + threadIdx.x;
  if (e >= a.Ncap) return;
  const int64_t n_vis = visible_entries(a.pos, qi, a.ratio, a.Ncap);
  float* srow = a.scores + qi * a.Ncap;
  if (e >= n_vis) { srow[e] = -INFINITY; return; }
  const int64_t row = (int64_t(b) * a.Ncap + e) * D;
  float sc = 0.f;
  for (int h = 0; h < H; ++h) {
    float dot = 0.f;
    for (int d = 0; d < D; ++d) dot += qs[h * D + d] * load_elem(a.cache, a.dtype, row + d);
    sc += fmaxf(dot, 0.f) * qs[H * D + h];
  }
  srow[e] = sc;
}

}  // namespace

hipError_t launch_index_score(const IndexArgs& a, hipStream_t stream) {
  const int64_t nq = int64_t(a.B) * a.S;
  if (nq == 0 || a.Ncap == 0) return hipSuccess;
  if (a.use_mfma && a.H == kHI && a.D == kDI) {
    const dim3 grid(unsigned(nq), (a.Ncap + kStreamBlockRows - 1) / kStreamBlockRows);
    hipLaunchKernelGGL(index_stream, grid, dim3(kWave * kStreamWaves), 0, stream, a);
  } else {
    const dim3 grid(unsigned(nq), (a.Ncap + 255) / 256);
    hipLaunchKernelGGL(index_any, grid, dim3(256), (a.H * a.D + a.H) * sizeof(float), stream, a);
  }
  return hipGetLastError();
}

}  // namespace csa
