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
//    from HBM into registers (every load instruction covers 64 contiguous
//    bytes of 16 rows), 4 x 16x16x32 MFMA per 16 rows and K-step, then ReLU,
//    head weights and a two-step cross-lane sum.
//  * index_tile (many queries per sequence, e.g. prefill): a workgroup stages
//    512 index rows in LDS once; each wave then scores its own queries
//    against them without further barriers, stopping at each query's causal
//    bound.
//
// A and B share the K order of a K-step: lane group g, element i <-> dim
// ks*32 + g*8 + i.
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
// Streaming kernel: grid (B*S, ceil(Ncap / (512*STEPS))), 8 waves.
// Block rows come in steps of 512 (64 per wave); step s+1 is loaded while
// step s is multiplied.  The query operand (16 KiB) is staged once per block
// in LDS and then held in VGPRs by every wave.
// ---------------------------------------------------------------------------
constexpr int kStreamWaves = 8;
constexpr int kStepRows = kStreamWaves * 64;

template <int STEPS>
__global__ __launch_bounds__(kWave* kStreamWaves) void index_stream(IndexArgs a) {
  __shared__ uint4 qs[kHI * (kDI / 8 + 1)];
  __shared__ float wsh[kHI];
  const int64_t qi = blockIdx.x;
  const int b = int(qi / a.S);
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int g = lane / 16, r16 = lane % 16;
  const int Ncap = a.Ncap;
  const int64_t n_vis = visible_entries(a.pos, qi, a.ratio, Ncap);
  const int64_t row0 = int64_t(blockIdx.y) * kStepRows * STEPS;
  float* srow = a.scores + qi * Ncap;

  if (row0 >= n_vis) {  // nothing visible in this block
    for (int64_t e = row0 + tid; e < row0 + int64_t(kStepRows) * STEPS && e < Ncap; e += kWave * kStreamWaves)
      srow[e] = -INFINITY;
    return;
  }
  const uint16_t* cache = static_cast<const uint16_t*>(a.cache) + int64_t(b) * Ncap * kDI;
  // per 16-row block and K-step, lane (g, r16) reads row r16, bytes ks*64 + g*16:
  // every load instruction covers 64 contiguous bytes of 16 rows
  auto load = [&](int step, uint4 (&kb)[4][4]) {
    const int64_t base = row0 + int64_t(step) * kStepRows + wave * 64;
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) {
      const int64_t e = base + blk * 16 + r16;
      if (e < n_vis) {
        const uint4* src = reinterpret_cast<const uint4*>(cache + e * kDI) + g;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) kb[blk][ks] = src[ks * 4];
      } else {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) kb[blk][ks] = uint4{0, 0, 0, 0};
      }
    }
  };
  // the first step's rows are requested before the query operand is staged
  uint4 kb0[4][4];
  load(0, kb0);
  {
    const uint4* q = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.q_idx) + qi * (kHI * kDI));
    for (int i = tid; i < kHI * kDI / 8; i += kWave * kStreamWaves) qs[(i / (kDI / 8)) * (kDI / 8 + 1) + i % (kDI / 8)] = q[i];
    if (tid < kHI) wsh[tid] = a.w[qi * kHI + tid];
  }
  __syncthreads();
  bf16x8 qa[4][4];  // [head tile][K-step]: Q[mt*16 + r16][ks*32 + g*8 .. +7]
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qa[mt][ks] = as_bf16x8(qs[(mt * 16 + r16) * (kDI / 8 + 1) + ks * 4 + g]);
  float wv[4][4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) wv[mt][i] = wsh[mt * 16 + g * 4 + i];

  auto score = [&](int step, const uint4 (&kb)[4][4]) {
    const int64_t base = row0 + int64_t(step) * kStepRows + wave * 64;
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
        for (int i = 0; i < 4; ++i) part += relu(acc[mt][i]) * wv[mt][i];
      part += __shfl_xor(part, 16, kWave);
      part += __shfl_xor(part, 32, kWave);
      const int64_t e = base + blk * 16 + r16;
      if (g == 0 && e < Ncap) srow[e] = e < n_vis ? part : -INFINITY;
    }
  };
  if constexpr (STEPS == 1) {
    score(0, kb0);
  } else {
    uint4 kb1[4][4];
#pragma unroll
    for (int s = 0; s < STEPS; s += 2) {
      if (s + 1 < STEPS) load(s + 1, kb1);
      score(s, kb0);
      if (s + 1 < STEPS) {
        if (s + 2 < STEPS) load(s + 2, kb0);
        score(s + 1, kb1);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Tile kernel (many queries per sequence, e.g. prefill): grid 1-D, 8 waves.
// A block owns 32 queries x 512 index rows.  The rows are staged once into
// LDS (row pitch padded by 32 bytes so that the 16 rows of a fragment sit on
// different banks); after that single barrier every wave runs on its own:
// it holds one query's 64x128 operand in VGPRs (the next query's operand in
// flight), streams 16-row tiles of the block's rows from LDS as MFMA B
// operands, and stops at the query's causal bound.  The entry tiles of one
// query chunk go to one XCD back to back (workgroups are dealt round-robin
// over the 8 XCDs), so a chunk's query operands come from HBM once and then
// from that XCD's L2.
// ---------------------------------------------------------------------------
constexpr int kTileQ = 32;
constexpr int kTileE = 512;
constexpr int kXcd = 8;
constexpr int kRowVec = kDI / 8;      // uint4 per index row
constexpr int kRowPitch = kRowVec + 2;  // 288 B: 16 rows of one 16-byte column fall on distinct banks

constexpr int kNT = 2;  // 16-row tiles per MFMA step of the tile kernel

__global__ __launch_bounds__(kWave* kStreamWaves) void index_tile(IndexArgs a, int qchunks_per_seq, int etiles,
                                                                 int nchunks) {
  __shared__ uint4 rows[kTileE * kRowPitch];
  __shared__ float wsh[kTileQ][kHI];
  __shared__ int svis[kTileQ];
  constexpr int kThreads = kWave * kStreamWaves;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int g = lane / 16, r16 = lane % 16;
  const int xcd = blockIdx.x % kXcd, local = blockIdx.x / kXcd;
  const int chunk = (local / etiles) * kXcd + xcd;
  const int tile = local % etiles;
  if (chunk >= nchunks) return;
  const int b = chunk / qchunks_per_seq;
  const int s0 = (chunk % qchunks_per_seq) * kTileQ;
  const int nq = min(kTileQ, a.S - s0);
  const int64_t q0 = int64_t(b) * a.S + s0;
  const int Ncap = a.Ncap;
  const int e_blk = tile * kTileE;
  const int e_end = min(e_blk + kTileE, Ncap);
  if (tid < kTileQ) svis[tid] = tid < nq ? int(visible_entries(a.pos, q0 + tid, a.ratio, Ncap)) : 0;
  __syncthreads();
  int vmax = 0;
  for (int j = 0; j < nq; ++j) vmax = max(vmax, svis[j]);
  if (e_blk >= vmax) {  // no query of the chunk sees any row of the tile
    for (int j = 0; j < nq; ++j)
      for (int e = e_blk + tid; e < e_end; e += kThreads) a.scores[(q0 + j) * Ncap + e] = -INFINITY;
    return;
  }
  // stage the visible part of the block's rows
  {
    const int n_rows = min(e_end, vmax) - e_blk;
    const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.cache) +
                                                      (int64_t(b) * Ncap + e_blk) * kDI);
    for (int i = tid; i < n_rows * kRowVec; i += kThreads) rows[(i / kRowVec) * kRowPitch + i % kRowVec] = src[i];
    for (int i = tid; i < nq * kHI; i += kThreads) wsh[i / kHI][i % kHI] = a.w[q0 * kHI + i];
  }
  __syncthreads();

  const uint4* qsrc = reinterpret_cast<const uint4*>(a.q_idx);
  auto fetch = [&](int j, bf16x8 (&dst)[4][4]) {
    const uint4* q = qsrc + (q0 + j) * (kHI * kRowVec);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) dst[mt][ks] = as_bf16x8(q[(mt * 16 + r16) * kRowVec + ks * 4 + g]);
  };
  auto score_query = [&](int j, const bf16x8 (&qa)[4][4]) {
    const float* wq = wsh[j] + g * 4;
    const int nv = svis[j];
    float* srow = a.scores + (q0 + j) * Ncap;
    const int e_vis = min(e_end, nv);  // rows [e_blk, e_vis) are scored, the rest of the tile is -inf
    for (int e = max(e_vis, e_blk) + lane; e < e_end; e += kWave) srow[e] = -INFINITY;
    // kNT 16-row tiles (4*kNT independent accumulator chains) per step keep
    // the matrix pipe fed; the ReLU / weight epilogue follows each step
    for (int t0 = e_blk; t0 < e_vis; t0 += kNT * 16) {
      floatx4 acc[kNT][4];  // [16-row tile][head tile]
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) acc[nt][mt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) {
          const bf16x8 kk = as_bf16x8(rows[(t0 - e_blk + nt * 16 + r16) * kRowPitch + g + ks * 4]);
#pragma unroll
          for (int mt = 0; mt < 4; ++mt)
            acc[nt][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[mt][ks], kk, acc[nt][mt], 0, 0, 0);
        }
      }
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) {
        float part = 0.f;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          const float4 w4 = *reinterpret_cast<const float4*>(wq + mt * 16);
          part += relu(acc[nt][mt][0]) * w4.x;
          part += relu(acc[nt][mt][1]) * w4.y;
          part += relu(acc[nt][mt][2]) * w4.z;
          part += relu(acc[nt][mt][3]) * w4.w;
        }
        part += __shfl_xor(part, 16, kWave);
        part += __shfl_xor(part, 32, kWave);
        const int e = t0 + nt * 16 + r16;
        if (g == 0 && e < e_end) srow[e] = e < nv ? part : -INFINITY;
      }
    }
  };
  // wave w takes queries w, w+8, ...; two operand sets alternate so that the
  // next query's operand is in flight while the current one is scored
  bf16x8 qa0[4][4], qa1[4][4];
  int j = wave;
  if (j < nq) fetch(j, qa0);
  while (j < nq) {
    if (j + kStreamWaves < nq) fetch(j + kStreamWaves, qa1);
    score_query(j, qa0);
    j += kStreamWaves;
    if (j >= nq) break;
    if (j + kStreamWaves < nq) fetch(j + kStreamWaves, qa0);
    score_query(j, qa1);
    j += kStreamWaves;
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
  if (a.use_mfma && a.H == kHI && a.D == kDI && a.S >= 2 * kTileQ) {
    const int qcs = (a.S + kTileQ - 1) / kTileQ;
    const int nchunks = a.B * qcs;
    const int etiles = (a.Ncap + kTileE - 1) / kTileE;
    const int64_t nblocks = int64_t((nchunks + kXcd - 1) / kXcd) * kXcd * etiles;
    hipLaunchKernelGGL(index_tile, dim3(unsigned(nblocks)), dim3(kWave * kStreamWaves), 0, stream, a, qcs, etiles,
                       nchunks);
  } else if (a.use_mfma && a.H == kHI && a.D == kDI) {
    const int64_t blocks1 = nq * ((a.Ncap + kStepRows - 1) / kStepRows);
    if (blocks1 <= 4096) {
      const dim3 grid(unsigned(nq), (a.Ncap + kStepRows - 1) / kStepRows);
      hipLaunchKernelGGL(index_stream<1>, grid, dim3(kWave * kStreamWaves), 0, stream, a);
    } else {
      constexpr int kSteps = 4;
      const dim3 grid(unsigned(nq), (a.Ncap + kStepRows * kSteps - 1) / (kStepRows * kSteps));
      hipLaunchKernelGGL(index_stream<kSteps>, grid, dim3(kWave * kStreamWaves), 0, stream, a);
    }
  } else {
    const dim3 grid(unsigned(nq), (a.Ncap + 255) / 256);
    hipLaunchKernelGGL(index_any, grid, dim3(256), (a.H * a.D + a.H) * sizeof(float), stream, a);
  }
  return hipGetLastError();
}

}  // namespace csa
