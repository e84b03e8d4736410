// Indexer scoring: score[e] = sum_h w[h] * relu(q_idx[h] . idx_cache[e]).
//
// "DeepSeek-V4-Flash 架构：一个 token 的旅程", section "少读 KV 之前，Indexer
// 仍要给历史打分" (64 heads of dim 128 over one shared 128-d index cache,
// signed weights); "Lab tổng hợp DeepSeek-V4.1-Flash", section "3 Giải pháp"
// (ReLU on each head's dot product).
//
// Every 256-byte index row meets 64 heads x 128 dims: 64 flop per byte, more
// than a vector-ALU roofline can stream at HBM rate, so the 64 heads form the
// M side of a bf16 matrix-core product even for a single query.  Kernels:
//
//  * index_stream (few queries over short caches, e.g. a 64K-token decode):
//    each wave keeps the query's 64x128 operand in registers and loads its
//    64 index rows straight from HBM into registers (every load instruction
//    covers 64 contiguous bytes of 16 rows), 4 x 16x16x32 MFMA per 16 rows
//    and K-step, then ReLU, head weights and a two-step cross-lane sum.
//  * index_flat (up to 1,024 queries over >= 2M rows in all, e.g. a 1M-token
//    decode batch): one persistent workgroup per CU; every wave streams an
//    equal share of all queries' visible rows through a private LDS ring.
//  * index_dma (more queries over long caches): the same ring per wave over
//    a fixed row range of one query.
//  * index_tile (many queries per sequence, e.g. prefill): the query
//    operands stay in registers and the index rows stream past them through
//    LDS up to the workgroup's causal bound.
//  * index_any: other shapes and fp32, on the vector ALU.
//
// A and B share the K order of a K-step: lane group g, element i <-> dim
// ks*32 + g*8 + i.
#include "common.h"
#include "kernels.h"

namespace csa {
namespace {

constexpr int kHI = 64;   // indexer heads on the matrix-core path
constexpr int kDI = 128;  // indexer head dim on the matrix-core path
constexpr int kRowB = kDI * 2;  // bytes per index row

__device__ __forceinline__ int64_t visible_entries(const int* pos, int64_t qi, int ratio, int Ncap) {
  const int p = pos[qi];
  const int64_t nv = p >= 0 ? (int64_t(p) + 1) / ratio : 0;
  return nv < Ncap ? nv : Ncap;
}

typedef __attribute__((address_space(3))) void lds_void;
// One LDS copy instruction: lane l moves the 16 bytes at base + voff[l] to
// LDS address lds + 16 l (M0 carries lds).  The kernel waits for it itself.
// The asm supplies its own wait states (the compiler's hazard checks do not
// see into asm): 5 after a VALU write of the address SGPRs, 1 after the M0
// write.
__device__ __forceinline__ void copy_to_lds(const void* base, uint32_t voff, uint32_t lds) {
  const uint64_t r = reinterpret_cast<uint64_t>(base);
  const uint64_t su = uint64_t(uint32_t(__builtin_amdgcn_readfirstlane(uint32_t(r)))) |
                      (uint64_t(uint32_t(__builtin_amdgcn_readfirstlane(uint32_t(r >> 32)))) << 32);
  asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(su), "{m0}"(lds) : "memory");
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
  // The query operand (16 KiB, L2 hits when nothing else is in flight) is
  // requested before anything else and staged in LDS before any row is
  // requested.  Requested beside the rows, it waited behind the row traffic
  // of the whole chip (an L2 hit then took 1-5 us instead of 0.2-0.6), and
  // no product could start before it.
  // (two named registers per thread: an array here would be placed in LDS,
  // whose store would then wait for the loads)
  static_assert(kHI * kDI / 8 == 2 * kWave * kStreamWaves, "two operand slots per thread");
  const uint4* qg = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.q_idx) + qi * (kHI * kDI));
  const int i0 = tid, i1 = tid + kWave * kStreamWaves;
  const uint4 qv0 = qg[i0], qv1 = qg[i1];
  const float wq = a.w[qi * kHI + tid % kHI];  // (every lane loads: no branch around the load)
  __builtin_amdgcn_sched_barrier(0);
  const int64_t n_vis = visible_entries(a.pos, qi, a.ratio, Ncap);
  const int64_t row0 = int64_t(blockIdx.y) * kStepRows * STEPS;
  float* srow = a.scores + qi * Ncap;

  if (row0 >= n_vis) {  // nothing visible in this block
    for (int64_t e = row0 + tid; e < row0 + int64_t(kStepRows) * STEPS && e < Ncap; e += kWave * kStreamWaves)
      srow[e] = -INFINITY;
    return;
  }
  const uint16_t* cache = static_cast<const uint16_t*>(a.cache) + (a.pt.pages ? 0 : int64_t(b) * Ncap * kDI);
  // per 16-row block and K-step, lane (g, r16) reads row r16, bytes ks*64 + g*16:
  // every load instruction covers 64 contiguous bytes of 16 rows
  auto load = [&](int step, uint4 (&kb)[4][4]) {
    const int64_t base = row0 + int64_t(step) * kStepRows + wave * 64;
    // rows past the causal bound repeat the last visible row (finite, their
    // scores are masked): every lane issues the same loads, so the counts of
    // loads in flight are static and the operand's wait below stays short
    const int64_t last = n_vis - 1;
    // a paged cache: the wave's 64 rows share one page (pages hold a
    // multiple of 64 rows); shift the base so that row e reads its pool row
    const uint16_t* cb = cache;
    if (a.pt.pages) {
      const int64_t lp = (base < last ? base : last) >> a.pt.page_shift;
      const int pg = a.pt.pages[int64_t(b) * a.pt.max_pages + lp];
      // an unallocated or foreign page reads the pool's first page instead
      // (its scores are still written; such a table is the caller's error)
      cb = cache + ((int64_t(pg >= 0 && pg < a.pt.pool_pages ? pg : 0) - lp) << a.pt.page_shift) * kDI;
    }
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) {
      const int64_t e = base + blk * 16 + r16;
      const uint4* src = reinterpret_cast<const uint4*>(cb + (e < last ? e : last) * kDI) + g;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) kb[blk][ks] = src[ks * 4];
    }
  };
  qs[(i0 / (kDI / 8)) * (kDI / 8 + 1) + i0 % (kDI / 8)] = qv0;
  qs[(i1 / (kDI / 8)) * (kDI / 8 + 1) + i1 % (kDI / 8)] = qv1;
  if (tid < kHI) wsh[tid] = wq;
  __syncthreads();
  // then the first step's rows, scored block by block as they land
  uint4 kb0[4][4];
  load(0, kb0);
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
      part = sum_rows4(part);
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
// Tile kernel (many queries per sequence, e.g. prefill): grid 1-D, 4 waves,
// three workgroups per CU.  A workgroup owns 4 consecutive queries of one
// sequence; wave w keeps query w's 64x128 operand in VGPRs for the whole run
// and the index rows stream past it through LDS in chunks of 64 rows
// (copied HBM -> LDS by the load unit, double-buffered), up to the largest
// causal bound of the 4 queries.  Each K fragment read from LDS feeds the 4
// head tiles of the wave's query.  LDS rows are 256 B with 16-byte chunk c of
// row r stored at chunk c ^ (r % 16), so the 16 rows of one fragment fall on
// distinct banks.  Scores are staged in LDS and written one chunk later as
// coalesced 16-byte stores.  Workgroups are taken heaviest first (the last
// queries see the most rows).
// ---------------------------------------------------------------------------
constexpr int kTQ = 4;          // queries per workgroup (one per wave)
constexpr int kTWaves = 4;
constexpr int kTThreads = kTWaves * kWave;
constexpr int kCR = 64;         // index rows per chunk
constexpr int kCopyPerWave = kCR / kTWaves / 4;  // 4 rows per LDS copy instruction

__global__ __launch_bounds__(kTThreads, 3) void index_tile(IndexArgs a, int groups_per_seq, int ngroups) {
  __shared__ __attribute__((aligned(16))) unsigned char rows[2][kCR * kRowB];
  __shared__ __attribute__((aligned(16))) float sc[2][kTWaves][kCR];
  __shared__ int svis[kTQ];
  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int g = lane / 16, r16 = lane % 16;
  const int grp = ngroups - 1 - int(blockIdx.x);  // heaviest first
  const int b = grp / groups_per_seq;
  const int s0 = (grp % groups_per_seq) * kTQ;
  const int nq = min(kTQ, a.S - s0);
  const int64_t q0 = int64_t(b) * a.S + s0;
  const int Ncap = a.Ncap;
  if (tid < kTQ) svis[tid] = tid < nq ? int(visible_entries(a.pos, q0 + tid, a.ratio, Ncap)) : 0;
  __syncthreads();
  int vmax = 0;
  for (int j = 0; j < nq; ++j) vmax = max(vmax, svis[j]);
  const int n_chunks = (vmax + kCR - 1) / kCR;
  const uint16_t* cache = static_cast<const uint16_t*>(a.cache) + int64_t(b) * Ncap * kDI;
  const uint32_t lds_rows = uint32_t(reinterpret_cast<uintptr_t>((lds_void*)&rows[0][0]));
  // wave w copies rows 16w..16w+15 of a chunk, 4 rows per instruction; rows
  // past the causal bound repeat the last visible row (finite, masked)
  auto issue = [&](int c, int buf) {
#pragma unroll
    for (int u = 0; u < kCopyPerWave; ++u) {
      const int rl = wave * (kCR / kTWaves) + u * 4 + g;  // row of this lane within the chunk
      const int e = min(c * kCR + rl, vmax - 1);
      const uint32_t voff = uint32_t(e) * kRowB + uint32_t(((r16 ^ (rl & 15)) << 4));
      copy_to_lds(cache, voff, lds_rows + uint32_t(buf * kCR * kRowB + (wave * (kCR / kTWaves) + u * 4) * kRowB));
    }
  };
  if (n_chunks > 0) issue(0, 0);

  // this wave's query (an absent one reuses query 0's operands; its scores are never stored)
  const int nv = wave < nq ? svis[wave] : 0;
  const int64_t qw = q0 + (wave < nq ? wave : 0);
  bf16x8 qa[4][4];  // [head tile][K-step]: Q[mt*16 + r16][ks*32 + g*8 .. +7]
  float wv[4][4];   // [head tile][i]: w[mt*16 + g*4 + i]
  {
    const uint4* q = reinterpret_cast<const uint4*>(a.q_idx) + qw * (kHI * kDI / 8);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) qa[mt][ks] = as_bf16x8(q[(mt * 16 + r16) * (kDI / 8) + ks * 4 + g]);
      const float4 w4 = *reinterpret_cast<const float4*>(a.w + qw * kHI + mt * 16 + g * 4);
      wv[mt][0] = w4.x; wv[mt][1] = w4.y; wv[mt][2] = w4.z; wv[mt][3] = w4.w;
    }
  }
  // K fragment offsets within a 16-row tile: row r16, chunk (ks*4 + g) ^ r16
  int koff[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) koff[ks] = r16 * kRowB + (((ks * 4 + g) ^ r16) << 4);

  // scores of chunk c (staged in sc[c & 1]) go out at the start of chunk c+1:
  // lanes 0..15 store rows 4*lane .. +3 of the wave's query
  auto store_chunk = [&](int c) {
    const int rw = lane * 4;
    const int e = c * kCR + rw;
    if (lane < kCR / 4 && wave < nq && e < Ncap)
      *reinterpret_cast<float4*>(a.scores + qw * Ncap + e) = *reinterpret_cast<const float4*>(&sc[c & 1][wave][rw]);
  };

  for (int c = 0; c < n_chunks; ++c) {
    const int buf = c & 1;
    __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));  // vmcnt(0): chunk c's copies (and older stores) are done
    __syncthreads();  // every wave's copies landed; chunk c-1's buffer is free
    if (c + 1 < n_chunks) issue(c + 1, buf ^ 1);
    if (c > 0) store_chunk(c - 1);
    const unsigned char* tb = rows[buf];
    // The chunk's four 16-row tiles in one branch-free region: the MFMAs of
    // tile nt+1 are interleaved with the ReLU / weight epilogue of tile nt
    // (1 MFMA, then VALU work, ...), so the wave keeps issuing VALU while the
    // matrix core works.  Rows past the causal bound are scored too (copies of
    // a visible row) and masked to -inf.
    auto kload = [&](int nt, bf16x8 (&kk)[4]) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) kk[ks] = as_bf16x8(*reinterpret_cast<const uint4*>(tb + nt * 16 * kRowB + koff[ks]));
    };
    auto mma = [&](const bf16x8 (&kk)[4], floatx4 (&acc)[4]) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[mt][0], kk[0], floatx4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
      for (int ks = 1; ks < 4; ++ks)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[mt][ks], kk[ks], acc[mt], 0, 0, 0);
    };
    // lane holds heads mt*16 + g*4 + i of row c*kCR + nt*16 + r16
    auto epi = [&](int nt, const floatx4 (&acc)[4]) {
      float p4[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        p4[mt] = relu(acc[mt][0]) * wv[mt][0] + relu(acc[mt][1]) * wv[mt][1] + relu(acc[mt][2]) * wv[mt][2] +
                 relu(acc[mt][3]) * wv[mt][3];
      const float part = sum_rows4((p4[0] + p4[1]) + (p4[2] + p4[3]));
      if (g == 0) sc[buf][wave][nt * 16 + r16] = c * kCR + nt * 16 + r16 < nv ? part : -INFINITY;
    };
    auto interleave = [&]() {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // then up to three VALU
      }
    };
    bf16x8 ka[4], kb[4];  // K operands of the next two tiles
    floatx4 acc0[4], acc1[4];
    kload(0, ka);
    kload(1, kb);
    mma(ka, acc0);
    kload(2, ka);
    mma(kb, acc1);
    epi(0, acc0);
    interleave();
    kload(3, kb);
    mma(ka, acc0);
    epi(1, acc1);
    interleave();
    mma(kb, acc1);
    epi(2, acc0);
    interleave();
    epi(3, acc1);
  }
  if (n_chunks > 0) store_chunk(n_chunks - 1);
  // entries past the last chunk are invisible to every query of the group
  for (int j = 0; j < nq; ++j) {
    float* srow = a.scores + (q0 + j) * Ncap;
    for (int e = n_chunks * kCR + tid; e < Ncap; e += kTThreads) srow[e] = -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// LDS-streaming kernel (few queries per sequence, e.g. decode): grid
// (B*S, ceil(Ncap / (8*RW))), 8 waves, one workgroup per CU.  Wave w scores
// rows [row0 + w*RW, row0 + (w+1)*RW) on its own, with no workgroup barrier
// after the start: its rows come HBM -> LDS through a private four-slot ring
// of 16-row chunks (each copy instruction moves 4 whole rows, 1 KiB
// contiguous), three chunks copying while one is multiplied.  LDS rows are 256 B
// with 16-byte chunk c of row r stored at chunk c ^ (r % 16).  Scores collect
// in LDS and leave in 1 KiB stores at the end, so the copy waits never cover
// a store.
// ---------------------------------------------------------------------------
constexpr int kDW = 8;        // waves per workgroup
constexpr int kDChunk = 16;   // rows per ring slot
constexpr int kDSlots = 4;    // ring slots per wave (kDSlots - 1 chunks in flight)
constexpr int kDCopies = kDChunk / 4;  // copy instructions per chunk

template <int RW>
__global__ __launch_bounds__(kDW * kWave) void index_dma(IndexArgs a) {
  static_assert(RW % kDChunk == 0 && RW >= kDChunk, "rows per wave");
  __shared__ __attribute__((aligned(16))) unsigned char ring[kDW][kDSlots][kDChunk * kRowB];
  __shared__ __attribute__((aligned(16))) float sc[kDW][RW];
  __shared__ __attribute__((aligned(16))) float wsh[kHI];
  const int64_t qi = blockIdx.x;
  const int b = int(qi / a.S);
  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int g = lane / 16, r16 = lane % 16;
  const int Ncap = a.Ncap;
  const int n_vis = int(visible_entries(a.pos, qi, a.ratio, Ncap));
  const int row0 = int(blockIdx.y) * (kDW * RW);
  float* srow = a.scores + qi * Ncap;
  if (row0 >= n_vis) {  // nothing visible in this workgroup
    for (int e = row0 + tid; e < row0 + kDW * RW && e < Ncap; e += kDW * kWave) srow[e] = -INFINITY;
    return;
  }
  const int wr0 = row0 + wave * RW;  // this wave's first row
  const int wr_vis = n_vis - wr0;    // visible rows from wr0 on (may be <= 0)
  const int n_ch = wr_vis > 0 ? min(RW / kDChunk, (wr_vis + kDChunk - 1) / kDChunk) : 0;
  const uint16_t* cache = static_cast<const uint16_t*>(a.cache) + int64_t(b) * Ncap * kDI;
  const uint32_t ring_base = uint32_t(reinterpret_cast<uintptr_t>((lds_void*)&ring[wave][0][0]));
  // chunk ch of the wave: kDCopies copies of 4 rows; rows past the causal
  // bound repeat the last visible row (finite, masked)
  auto issue = [&](int ch) {
#pragma unroll
    for (int u = 0; u < kDCopies; ++u) {
      const int rl = u * 4 + g;
      const int e = min(wr0 + ch * kDChunk + rl, n_vis - 1);
      const uint32_t voff = uint32_t(e) * kRowB + uint32_t(((r16 ^ (rl & 15)) << 4));
      copy_to_lds(cache, voff, ring_base + uint32_t((ch % kDSlots) * kDChunk * kRowB + u * 4 * kRowB));
    }
  };
#pragma unroll
  for (int ch = 0; ch < kDSlots - 1; ++ch)
    if (ch < n_ch) issue(ch);
  if (tid < kHI) wsh[tid] = a.w[qi * kHI + tid];
  bf16x8 qa[4][4];  // [head tile][K-step]: Q[mt*16 + r16][ks*32 + g*8 .. +7]
  {
    const uint4* q = reinterpret_cast<const uint4*>(a.q_idx) + qi * (kHI * kDI / 8);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) qa[mt][ks] = as_bf16x8(q[(mt * 16 + r16) * (kDI / 8) + ks * 4 + g]);
  }
  __syncthreads();  // head weights
  float wv[4][4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) wv[mt][i] = wsh[mt * 16 + g * 4 + i];
  int koff[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) koff[ks] = r16 * kRowB + (((ks * 4 + g) ^ r16) << 4);

  for (int ch = 0; ch < n_ch; ++ch) {
    // this wave's copies of chunk ch are done (later chunks may be in flight)
    const int later = min(n_ch - 1 - ch, kDSlots - 2);
    if (later >= 2) __builtin_amdgcn_s_waitcnt((2 * kDCopies) | (7 << 4) | (15 << 8));
    else if (later == 1) __builtin_amdgcn_s_waitcnt(kDCopies | (7 << 4) | (15 << 8));
    else __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));
    const unsigned char* tb = &ring[wave][ch % kDSlots][0];
    {
      bf16x8 kk[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) kk[ks] = as_bf16x8(*reinterpret_cast<const uint4*>(tb + koff[ks]));
      floatx4 acc[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[mt][0], kk[0], floatx4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
      for (int ks = 1; ks < 4; ++ks)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[mt][ks], kk[ks], acc[mt], 0, 0, 0);
      float p4[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        p4[mt] = relu(acc[mt][0]) * wv[mt][0] + relu(acc[mt][1]) * wv[mt][1] + relu(acc[mt][2]) * wv[mt][2] +
                 relu(acc[mt][3]) * wv[mt][3];
      const float part = sum_rows4((p4[0] + p4[1]) + (p4[2] + p4[3]));
      const int rr = ch * kDChunk + r16;
      if (g == 0) sc[wave][rr] = rr < wr_vis ? part : -INFINITY;
    }
    // the slot's rows are consumed (their reads returned before the MFMAs)
    if (ch + kDSlots - 1 < n_ch) issue(ch + kDSlots - 1);
  }
  for (int rr = n_ch * kDChunk + lane; rr < RW; rr += kWave) sc[wave][rr] = -INFINITY;
  // the wave's scores, 256 rows per 16-byte store instruction
#pragma unroll
  for (int r4 = lane * 4; r4 < RW; r4 += kWave * 4)
    if (wr0 + r4 < Ncap) *reinterpret_cast<float4*>(srow + wr0 + r4) = *reinterpret_cast<const float4*>(&sc[wave][r4]);
}

// ---------------------------------------------------------------------------
// Balanced LDS-streaming kernel (decode): a persistent grid of one workgroup
// per CU, 8 waves.  The visible rows of all queries, cut into 16-row chunks,
// form one query-major list of C chunks; wave k of the W waves takes chunks
// [kC/W, (k+1)C/W), so every wave streams the same number of rows whatever
// the sequence lengths (a grid of equal row ranges per query leaves CUs idle
// at the end when lengths differ).  A wave streams its chunks through a
// private four-slot LDS ring as index_dma does, loads the next query's
// operands when its range enters that query, and gathers its scores 256 rows
// at a time.  A full buffer of scores is parked in registers (up to 16 per
// wave) and written once the wave's stream is done: score stores issued in
// the middle of the stream cost far more than their bytes (each one holds
// the wave's in-order load count until it is acknowledged, and the writes
// interleave with the row reads), about 9 % of the kernel at a 1M-token
// context.  Afterwards the workgroups share the -inf fill of every row past
// a query's last chunk.
// PAGED: the rows live in a page pool (pages of a power-of-two multiple of 64
// rows, so a 16-row chunk never straddles two); the issuing cursor keeps the
// pool page of its current logical page and, on entering a page, requests
// the next one's table entry, which arrives long before the cursor needs it.
// ---------------------------------------------------------------------------
constexpr int kFlatMaxQ = 1024;  // queries whose chunk counts fit in LDS
constexpr int kFlush = 256;      // score rows per store
constexpr int kSeg = 16;         // score segments a wave keeps until its stream ends

// s_waitcnt vmcnt(n) for a run-time n in 0..15
__device__ __forceinline__ void wait_vmem_upto15(int n) {
  switch (n) {
    case 0: __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8)); break;
    case 1: __builtin_amdgcn_s_waitcnt(1 | (7 << 4) | (15 << 8)); break;
    case 2: __builtin_amdgcn_s_waitcnt(2 | (7 << 4) | (15 << 8)); break;
    case 3: __builtin_amdgcn_s_waitcnt(3 | (7 << 4) | (15 << 8)); break;
    case 4: __builtin_amdgcn_s_waitcnt(4 | (7 << 4) | (15 << 8)); break;
    case 5: __builtin_amdgcn_s_waitcnt(5 | (7 << 4) | (15 << 8)); break;
    case 6: __builtin_amdgcn_s_waitcnt(6 | (7 << 4) | (15 << 8)); break;
    case 7: __builtin_amdgcn_s_waitcnt(7 | (7 << 4) | (15 << 8)); break;
    case 8: __builtin_amdgcn_s_waitcnt(8 | (7 << 4) | (15 << 8)); break;
    case 9: __builtin_amdgcn_s_waitcnt(9 | (7 << 4) | (15 << 8)); break;
    case 10: __builtin_amdgcn_s_waitcnt(10 | (7 << 4) | (15 << 8)); break;
    case 11: __builtin_amdgcn_s_waitcnt(11 | (7 << 4) | (15 << 8)); break;
    case 12: __builtin_amdgcn_s_waitcnt(12 | (7 << 4) | (15 << 8)); break;
    case 13: __builtin_amdgcn_s_waitcnt(13 | (7 << 4) | (15 << 8)); break;
    case 14: __builtin_amdgcn_s_waitcnt(14 | (7 << 4) | (15 << 8)); break;
    default: __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (15 << 8)); break;
  }
}

template <bool PAGED>
__global__ __launch_bounds__(kDW * kWave) void index_flat(IndexArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char ring[kDW][kDSlots][kDChunk * kRowB];
  __shared__ __attribute__((aligned(16))) float sc[kDW][kFlush];
  __shared__ int64_t cpre[kFlatMaxQ + 1];  // chunks of the queries before q
  __shared__ int64_t dpre[kFlatMaxQ + 1];  // 4-row groups past the chunks of the queries before q
  __shared__ int nvis_s[kFlatMaxQ];
  __shared__ int seg_meta[kDW][kSeg][3];  // query, first row, rows of each parked segment
  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int g = lane / 16, r16 = lane % 16;
  const int nq = a.B * a.S;
  const int Ncap = a.Ncap;

  // chunk and -inf-group counts of every query, scanned by wave 0
  if (wave == 0) {
    const int per = (nq + kWave - 1) / kWave;
    const int qb = lane * per;
    int64_t cs = 0, ds = 0;
    for (int j = 0; j < per; ++j) {
      const int q = qb + j;
      if (q < nq) {
        const int nv = int(visible_entries(a.pos, q, a.ratio, Ncap));
        nvis_s[q] = nv;
        const int ch = (nv + kDChunk - 1) / kDChunk;
        cs += ch;
        ds += Ncap > ch * kDChunk ? (Ncap - ch * kDChunk) / 4 : 0;
      }
    }
    int64_t ci = cs, di = ds;  // inclusive scans over lanes
    for (int o = 1; o < kWave; o <<= 1) {
      const int64_t cy = __shfl_up(ci, o, kWave), dy = __shfl_up(di, o, kWave);
      if (lane >= o) { ci += cy; di += dy; }
    }
    int64_t cx = ci - cs, dx = di - ds;
    for (int j = 0; j < per; ++j) {
      const int q = qb + j;
      if (q < nq) {
        cpre[q] = cx;
        dpre[q] = dx;
        const int nv = nvis_s[q];
        const int ch = (nv + kDChunk - 1) / kDChunk;
        cx += ch;
        dx += Ncap > ch * kDChunk ? (Ncap - ch * kDChunk) / 4 : 0;
      }
    }
    if (lane == kWave - 1) {
      cpre[nq] = ci;
      dpre[nq] = di;
    }
  }
  __syncthreads();

  // the query whose range holds list position c (prefix[q] <= c < prefix[q+1])
  auto find = [&](const int64_t* pre, int64_t c) -> int {
    int lo = 0, hi = nq;
    while (hi - lo > 1) {
      const int mid = (lo + hi) / 2;
      if (pre[mid] <= c) lo = mid;
      else hi = mid;
    }
    return lo;
  };
  struct Cur {
    int q, lc, nch, nv;  // query, its chunk, its chunk count, its visible rows
    int pq, plp, pg;     // (PAGED, issuing cursor) query and logical page of pool page pg
    int pnext;           // its table entry for logical page plp + 1 (requested, maybe in flight)
  };
  auto at = [&](int64_t c) -> Cur {
    Cur u;
    u.pq = -1;
    u.plp = -1;
    u.pg = 0;
    u.pnext = 0;
    u.q = __builtin_amdgcn_readfirstlane(find(cpre, c));
    u.lc = __builtin_amdgcn_readfirstlane(int(c - cpre[u.q]));
    u.nch = __builtin_amdgcn_readfirstlane(int(cpre[u.q + 1] - cpre[u.q]));
    u.nv = __builtin_amdgcn_readfirstlane(nvis_s[u.q]);
    return u;
  };
  auto advance = [&](Cur& u) {
    if (++u.lc < u.nch) return;
    u.lc = 0;
    do { ++u.q; } while (u.q < nq && __builtin_amdgcn_readfirstlane(int(cpre[u.q + 1] == cpre[u.q])));
    if (u.q < nq) {
      u.nch = __builtin_amdgcn_readfirstlane(int(cpre[u.q + 1] - cpre[u.q]));
      u.nv = __builtin_amdgcn_readfirstlane(nvis_s[u.q]);
    }
  };

  const int64_t C = cpre[nq];
  const int64_t W = int64_t(gridDim.x) * kDW;
  const int64_t k = int64_t(blockIdx.x) * kDW + wave;
  const int64_t c0 = k * C / W;
  const int n = int((k + 1) * C / W - c0);  // chunks of this wave
  const uint16_t* cache0 = static_cast<const uint16_t*>(a.cache);
  const uint32_t ring_base = uint32_t(reinterpret_cast<uintptr_t>((lds_void*)&ring[wave][0][0]));
  // chunk u into ring slot `slot`: 4 copies of 4 rows; rows past the causal
  // bound repeat the last visible row (finite, masked)
  // a table entry as a pool page; an unallocated or foreign page reads the
  // pool's first page instead (its scores are still written; such a table is
  // the caller's error)
  auto pool_page = [&](int pg) { return (pg >= 0 && pg < a.pt.pool_pages) ? pg : 0; };
  // (read through the constant address space: a scalar load, whose wait
  // leaves the ring copies in flight)
  auto table_entry = [&](int q, int lp) {
    const __attribute__((address_space(4))) int* t = (const __attribute__((address_space(4))) int*)a.pt.pages;
    return t[int64_t(q / a.S) * a.pt.max_pages + lp];
  };
  auto issue = [&](Cur& u, int slot) {
    const uint16_t* cache;
    int e_base = 0;  // first row of `cache`, in the query's entry numbering
    if constexpr (PAGED) {
      const int lp = (u.lc * kDChunk) >> a.pt.page_shift;
      if (u.q != u.pq || lp != u.plp) {
        const int pg = (u.q == u.pq && lp == u.plp + 1) ? u.pnext : table_entry(u.q, lp);
        u.pg = __builtin_amdgcn_readfirstlane(pool_page(pg));
        u.pq = u.q;
        u.plp = lp;
        if (int64_t(lp + 1) << a.pt.page_shift < u.nv) u.pnext = table_entry(u.q, lp + 1);
      }
      cache = cache0 + (int64_t(u.pg) << a.pt.page_shift) * kDI;
      e_base = lp << a.pt.page_shift;
    } else {
      cache = cache0 + int64_t(u.q / a.S) * Ncap * kDI;
    }
#pragma unroll
    for (int cp = 0; cp < kDCopies; ++cp) {
      const int rl = cp * 4 + g;
      const int e = min(u.lc * kDChunk + rl, u.nv - 1) - e_base;
      const uint32_t voff = uint32_t(e) * kRowB + uint32_t(((r16 ^ (rl & 15)) << 4));
      copy_to_lds(cache, voff, ring_base + uint32_t(slot * kDChunk * kRowB + cp * 4 * kRowB));
    }
  };

  if (n > 0) {
    Cur ci = at(c0), cc = ci;
    for (int j = 0; j < kDSlots - 1 && j < n; ++j) {
      issue(ci, j);
      advance(ci);
    }
    bf16x8 qa[4][4];  // [head tile][K-step]: Q[mt*16 + r16][ks*32 + g*8 .. +7]
    float wv[4][4];
    int q_loaded = -1;
    int koff[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) koff[ks] = r16 * kRowB + (((ks * 4 + g) ^ r16) << 4);
    int sq = cc.q, sb = cc.lc * kDChunk, cnt = 0;  // buffered scores: rows sb .. sb+cnt-1 of query sq
    int f1 = 0, f2 = 0;                            // stores issued in the previous two iterations
    float4 seg[kSeg];
    int nseg = 0;
    // park the buffered scores in a register segment (no memory traffic), or
    // store them when every segment is taken; true if a store was issued
    auto flush = [&]() -> bool {
      const float4 v = *reinterpret_cast<const float4*>(&sc[wave][4 * lane]);
      if (nseg < kSeg) {
#pragma unroll
        for (int t = 0; t < kSeg; ++t)
          if (t == nseg) seg[t] = v;
        if (lane == 0) {
          seg_meta[wave][nseg][0] = sq;
          seg_meta[wave][nseg][1] = sb;
          seg_meta[wave][nseg][2] = cnt;
        }
        ++nseg;
        return false;
      }
      if (4 * lane < cnt && sb + 4 * lane < Ncap)
        *reinterpret_cast<float4*>(a.scores + int64_t(sq) * Ncap + sb + 4 * lane) = v;
      return true;
    };
    for (int j = 0; j < n; ++j) {
      // chunk j's copies are done; what was issued after them may still fly:
      // the stores of the two previous iterations and up to two later chunks
      wait_vmem_upto15(f1 + f2 + kDCopies * ((j + 1 < n) + (j + 2 < n)));
      if (cc.q != q_loaded) {  // first chunk of a query in this range
        q_loaded = cc.q;
        const uint4* qp = reinterpret_cast<const uint4*>(a.q_idx) + int64_t(q_loaded) * (kHI * kDI / 8);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) qa[mt][ks] = as_bf16x8(qp[(mt * 16 + r16) * (kDI / 8) + ks * 4 + g]);
        const float* wq = a.w + int64_t(q_loaded) * kHI;  // w is only 4-byte aligned
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) wv[mt][i] = wq[mt * 16 + g * 4 + i];
      }
      const unsigned char* tb = &ring[wave][j % kDSlots][0];
      bf16x8 kk[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) kk[ks] = as_bf16x8(*reinterpret_cast<const uint4*>(tb + koff[ks]));
      floatx4 acc[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[mt][0], kk[0], floatx4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
      for (int ks = 1; ks < 4; ++ks)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[mt][ks], kk[ks], acc[mt], 0, 0, 0);
      float p4[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        p4[mt] = relu(acc[mt][0]) * wv[mt][0] + relu(acc[mt][1]) * wv[mt][1] + relu(acc[mt][2]) * wv[mt][2] +
                 relu(acc[mt][3]) * wv[mt][3];
      const float part = sum_rows4((p4[0] + p4[1]) + (p4[2] + p4[3]));
      // scores leave when the buffer is full or the chunk starts another query
      int f0 = 0;
      if (cnt > 0 && (cc.q != sq || cnt == kFlush)) {
        f0 = flush() ? 1 : 0;
        sq = cc.q;
        sb = cc.lc * kDChunk;
        cnt = 0;
      }
      const int e = cc.lc * kDChunk + r16;
      if (g == 0) sc[wave][cnt + r16] = e < cc.nv ? part : -INFINITY;
      cnt += kDChunk;
      f2 = f1;
      f1 = f0;
      advance(cc);
      // the slot of chunk j is consumed (its reads returned before the MFMAs)
      if (j + kDSlots - 1 < n) {
        issue(ci, (j + kDSlots - 1) % kDSlots);
        advance(ci);
      }
    }
    flush();
    // the parked segments leave together once the stream is done
#pragma unroll
    for (int t = 0; t < kSeg; ++t) {
      if (t < nseg) {
        const int q = seg_meta[wave][t][0], e0 = seg_meta[wave][t][1], m = seg_meta[wave][t][2];
        if (4 * lane < m && e0 + 4 * lane < Ncap)
          *reinterpret_cast<float4*>(a.scores + int64_t(q) * Ncap + e0 + 4 * lane) = seg[t];
      }
    }
  }

  // -inf past every query's last chunk, in float4 groups shared by all workgroups
  const int64_t D4 = dpre[nq];
  const int64_t u0 = int64_t(blockIdx.x) * D4 / gridDim.x, u1 = (int64_t(blockIdx.x) + 1) * D4 / gridDim.x;
  for (int64_t u = u0 + tid; u < u1; u += kDW * kWave) {
    const int q = find(dpre, u);
    const int64_t e = int64_t((nvis_s[q] + kDChunk - 1) / kDChunk) * kDChunk + 4 * (u - dpre[q]);
    *reinterpret_cast<float4*>(a.scores + int64_t(q) * Ncap + e) = float4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
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
  const int64_t prow = a.pt.pages ? paged_row(a.pt, b, e) : int64_t(b) * a.Ncap + e;
  if (prow < 0) { srow[e] = -INFINITY; return; }  // a paged entry without a page of the pool
  const int64_t row = prow * D;
  float sc = 0.f;
  for (int h = 0; h < H; ++h) {
    float dot = 0.f;
    for (int d = 0; d < D; ++d) dot += qs[h * D + d] * load_elem(a.cache, a.dtype, row + d);
    sc += fmaxf(dot, 0.f) * qs[H * D + h];
  }
  srow[e] = sc;
}

}  // namespace

// Compute units of the current device (the persistent grid size), looked up
// once per device.
int cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

hipError_t launch_index_score(const IndexArgs& a, hipStream_t stream) {
  const int64_t nq = int64_t(a.B) * a.S;
  if (nq == 0 || a.Ncap == 0) return hipSuccess;
  const bool paged = a.pt.pages != nullptr;  // paged caches: the streaming kernels or the vector path
  if (!paged && a.use_mfma && a.H == kHI && a.D == kDI && a.S >= 2 * kTQ && a.Ncap % 4 == 0) {
    const int gps = (a.S + kTQ - 1) / kTQ;
    const int ngroups = a.B * gps;
    hipLaunchKernelGGL(index_tile, dim3(unsigned(ngroups)), dim3(kTThreads), 0, stream, a, gps, ngroups);
  } else if (a.use_mfma && a.H == kHI && a.D == kDI && a.Ncap % 4 == 0 && nq <= kFlatMaxQ &&
             nq * int64_t(a.Ncap) >= (int64_t(1) << 21)) {
    // long caches (>= 2M rows in all): balanced persistent streaming
    if (paged) hipLaunchKernelGGL(index_flat<true>, dim3(unsigned(cu_count())), dim3(kDW * kWave), 0, stream, a);
    else hipLaunchKernelGGL(index_flat<false>, dim3(unsigned(cu_count())), dim3(kDW * kWave), 0, stream, a);
  } else if (!paged && a.use_mfma && a.H == kHI && a.D == kDI && a.Ncap % 4 == 0 &&
             nq * int64_t(a.Ncap) >= (int64_t(1) << 21)) {
    // long caches of more queries than index_flat's prefix holds: rows per
    // wave the smallest of 32 .. 512 that keeps the grid within 2048 workgroups
    const int64_t rows = nq * int64_t(a.Ncap);
    int rw = 32;
    while (rw < 512 && rows > int64_t(2048) * kDW * rw) rw *= 2;
    const dim3 grid(unsigned(nq), unsigned((a.Ncap + kDW * rw - 1) / (kDW * rw)));
    const dim3 block(kDW * kWave);
    switch (rw) {
      case 32: hipLaunchKernelGGL(index_dma<32>, grid, block, 0, stream, a); break;
      case 64: hipLaunchKernelGGL(index_dma<64>, grid, block, 0, stream, a); break;
      case 128: hipLaunchKernelGGL(index_dma<128>, grid, block, 0, stream, a); break;
      case 256: hipLaunchKernelGGL(index_dma<256>, grid, block, 0, stream, a); break;
      default: hipLaunchKernelGGL(index_dma<512>, grid, block, 0, stream, a); break;
    }
  } else if (a.use_mfma && a.H == kHI && a.D == kDI) {
    // one step per workgroup while that still gives few workgroups per CU;
    // long caches run many steps per workgroup, so that fewer workgroups pay
    // the start-up latency
    const int64_t blocks1 = nq * ((a.Ncap + kStepRows - 1) / kStepRows);
    if (blocks1 <= 4096) {
      const dim3 grid(unsigned(nq), (a.Ncap + kStepRows - 1) / kStepRows);
      hipLaunchKernelGGL(index_stream<1>, grid, dim3(kWave * kStreamWaves), 0, stream, a);
    } else if (blocks1 <= 8192) {
      constexpr int kSteps = 4;
      const dim3 grid(unsigned(nq), (a.Ncap + kStepRows * kSteps - 1) / (kStepRows * kSteps));
      hipLaunchKernelGGL(index_stream<kSteps>, grid, dim3(kWave * kStreamWaves), 0, stream, a);
    } else {
      constexpr int kSteps = 16;
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
