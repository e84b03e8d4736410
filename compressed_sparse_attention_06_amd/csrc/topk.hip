// Top-k selection of indexer scores.
//
// "DeepSeek-V4-Flash 架构：一个 token 的旅程", section "少读 KV 之前，Indexer
// 仍要给历史打分" (top-k fixes what the main attention reads) and "LLM Atlas:
// DeepSeek" §19 (k = 512 for Flash, 1024 for Pro).
//
// Scores map to order-preserving 32-bit keys (invisible / -inf -> 0).  A
// workgroup stages up to M keys of one row in LDS and finds the exact k-th
// largest key with four 8-bit radix passes (LDS histogram, suffix scan).  The
// kept set is then written by an ordered compaction: every thread owns a
// contiguous run of positions, two block scans give each thread its output
// offset and its share of the threshold-equal keys, so ties go to the lowest
// index and the output is sorted by index -- deterministic run to run.
//
// Rows longer than one LDS tile are cut into chunks; each chunk keeps its own
// top-k as (key, index) candidates, whose union provably holds the row's
// top-k under the same (key desc, index asc) order.  Candidate lists are
// reduced again until one tile remains.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace csa {
namespace {

constexpr int kMaxTile = 16384;

__device__ __forceinline__ uint32_t score_key(float f) {
  if (f == -INFINITY) return 0u;
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive scan over the block; returns the exclusive prefix, *total the sum.
template <int THREADS>
__device__ __forceinline__ uint32_t block_scan(uint32_t v, uint32_t* wsum, uint32_t* total) {
  constexpr int W = THREADS / kWave;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const uint32_t y = __shfl_up(x, o, kWave);
    if (lane >= o) x += y;
  }
  if (lane == kWave - 1) wsum[wave] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t run = 0;
    for (int i = 0; i < W; ++i) { const uint32_t t = wsum[i]; wsum[i] = run; run += t; }
    wsum[W] = run;
  }
  __syncthreads();
  const uint32_t ex = wsum[wave] + x - v;
  *total = wsum[W];
  __syncthreads();
  return ex;
}

struct SelectArgs {
  const float* scores;    // raw source: [R, N]
  const int* n_valid;     // raw source: [R] or null
  const uint32_t* ckey;   // candidate source: [R, in_len]
  const int* cidx;
  int in_len;             // raw: N; candidates: entries per row
  int k;
  int nchunks;            // chunks per row at this level (output stride)
  int* out_idx;           // final: [R, k]
  uint32_t* okey;         // chunked: [R, nchunks*k]
  int* oidx;
};

template <int THREADS, int ITEMS, bool FROM_CAND, bool FINAL>
__global__ __launch_bounds__(THREADS) void topk_select(SelectArgs a) {
  constexpr int M = THREADS * ITEMS;
  __shared__ uint32_t keys[M];
  __shared__ int idxs[FROM_CAND ? M : 1];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t wsum[THREADS / kWave + 1];
  __shared__ uint32_t pick[2];

  const int row = blockIdx.x, chunk = blockIdx.y, tid = threadIdx.x;
  const int64_t base = int64_t(chunk) * M;
  int len = a.in_len;
  if (!FROM_CAND && a.n_valid != nullptr) len = min(len, max(a.n_valid[row], 0));

  uint32_t ok = 0;
  for (int j = tid; j < M; j += THREADS) {
    const int64_t p = base + j;
    uint32_t key = 0;
    if (p < len) {
      if constexpr (FROM_CAND) {
        key = a.ckey[int64_t(row) * a.in_len + p];
        idxs[j] = a.cidx[int64_t(row) * a.in_len + p];
      } else {
        key = score_key(a.scores[int64_t(row) * a.in_len + p]);
      }
    }
    keys[j] = key;
    ok += key != 0u;
  }
  uint32_t n_ok;
  block_scan<THREADS>(ok, wsum, &n_ok);  // also orders the LDS fills

  uint32_t thr = 0, need_eq = 0;
  if (n_ok > uint32_t(a.k)) {
    uint32_t prefix = 0, mask = 0, remaining = a.k;
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int i = tid; i < 256; i += THREADS) hist[i] = 0;
      __syncthreads();
      for (int j = tid; j < M; j += THREADS) {
        const uint32_t key = keys[j];
        if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
      }
      __syncthreads();
      // suffix counts: cum[d] = #keys with this digit >= d
      const uint32_t hv = tid < 256 ? hist[255 - tid] : 0u;
      uint32_t tot;
      const uint32_t ex = block_scan<THREADS>(hv, wsum, &tot);
      if (tid < 256) {
        const int d = 255 - tid;
        const uint32_t above = ex, incl = ex + hv;  // digits > d, digits >= d
        if (incl >= remaining && above < remaining) { pick[0] = uint32_t(d); pick[1] = above; }
      }
      __syncthreads();
      remaining -= pick[1];
      prefix |= pick[0] << shift;
      mask |= 0xffu << shift;
      __syncthreads();
    }
    thr = prefix;
    need_eq = remaining;
  }

  // ordered compaction over contiguous runs of ITEMS positions
  const int j0 = tid * ITEMS;
  uint32_t gt = 0, eq = 0;
#pragma unroll
  for (int t = 0; t < ITEMS; ++t) {
    const uint32_t key = keys[j0 + t];
    gt += key > thr;
    eq += (key == thr) && (key != 0u);
  }
  uint32_t tot;
  const uint32_t p_eq = block_scan<THREADS>(eq, wsum, &tot);
  const uint32_t take = need_eq > p_eq ? min(need_eq - p_eq, eq) : 0u;
  uint32_t n_sel;
  uint32_t o = block_scan<THREADS>(gt + take, wsum, &n_sel);
  uint32_t taken = 0;
  const int64_t obase = FINAL ? int64_t(row) * a.k : (int64_t(row) * a.nchunks + chunk) * a.k;
#pragma unroll
  for (int t = 0; t < ITEMS; ++t) {
    const uint32_t key = keys[j0 + t];
    bool sel = key > thr;
    if (!sel && key == thr && key != 0u && taken < take) { sel = true; ++taken; }
    if (sel) {
      const int index = FROM_CAND ? idxs[j0 + t] : int(base + j0 + t);
      if constexpr (FINAL) {
        a.out_idx[obase + o] = index;
      } else {
        a.okey[obase + o] = key;
        a.oidx[obase + o] = index;
      }
      ++o;
    }
  }
  for (int i = int(n_sel) + tid; i < a.k; i += THREADS) {
    if constexpr (FINAL) {
      a.out_idx[obase + i] = -1;
    } else {
      a.okey[obase + i] = 0u;
      a.oidx[obase + i] = -1;
    }
  }
}

template <bool FROM_CAND, bool FINAL>
void launch_select(const SelectArgs& a, int len, int R, int nchunks, hipStream_t s) {
  const dim3 grid(R, nchunks);
  if (len <= 2048 && !FROM_CAND && nchunks == 1)
    hipLaunchKernelGGL((topk_select<256, 8, FROM_CAND, FINAL>), grid, dim3(256), 0, s, a);
  else if (len <= 8192 && nchunks == 1)
    hipLaunchKernelGGL((topk_select<512, 16, FROM_CAND, FINAL>), grid, dim3(512), 0, s, a);
  else
    hipLaunchKernelGGL((topk_select<1024, 16, FROM_CAND, FINAL>), grid, dim3(1024), 0, s, a);
}

int64_t chunks_of(int64_t len) { return (len + kMaxTile - 1) / kMaxTile; }

}  // namespace

TopkPlan plan_topk(int R, int N, int k) {
  TopkPlan p{0, 0, 0};
  int64_t len = N, maxlen = 0;
  while (len > kMaxTile) {
    len = chunks_of(len) * k;
    maxlen = std::max(maxlen, len);
    ++p.levels;
  }
  p.cand_elems = int64_t(R) * maxlen;
  p.ws_bytes = p.levels ? size_t(2) * size_t(p.cand_elems) * (sizeof(uint32_t) + sizeof(int)) : 0;
  return p;
}

hipError_t launch_topk(const float* scores, const int* n_valid, int R, int N, int k, int* idx, void* ws,
                       hipStream_t stream) {
  if (R == 0) return hipSuccess;
  const TopkPlan plan = plan_topk(R, N, k);
  SelectArgs a{};
  a.scores = scores;
  a.n_valid = n_valid;
  a.k = k;
  a.out_idx = idx;
  if (plan.levels == 0) {
    a.in_len = N;
    a.nchunks = 1;
    launch_select<false, true>(a, N, R, 1, stream);
    return hipGetLastError();
  }
  uint32_t* key_buf[2];
  int* idx_buf[2];
  char* w = static_cast<char*>(ws);
  for (int i = 0; i < 2; ++i) {
    key_buf[i] = reinterpret_cast<uint32_t*>(w);
    w += plan.cand_elems * sizeof(uint32_t);
    idx_buf[i] = reinterpret_cast<int*>(w);
    w += plan.cand_elems * sizeof(int);
  }
  // level 1: raw scores -> per-chunk candidates
  int64_t len = N;
  int nch = int(chunks_of(len));
  a.in_len = N;
  a.nchunks = nch;
  a.okey = key_buf[0];
  a.oidx = idx_buf[0];
  launch_select<false, false>(a, N, R, nch, stream);
  len = int64_t(nch) * k;
  int cur = 0;
  // further levels: candidates -> candidates
  while (len > kMaxTile) {
    nch = int(chunks_of(len));
    SelectArgs c{};
    c.ckey = key_buf[cur];
    c.cidx = idx_buf[cur];
    c.in_len = int(len);
    c.k = k;
    c.nchunks = nch;
    c.okey = key_buf[cur ^ 1];
    c.oidx = idx_buf[cur ^ 1];
    launch_select<true, false>(c, int(len), R, nch, stream);
    cur ^= 1;
    len = int64_t(nch) * k;
  }
  SelectArgs f{};
  f.ckey = key_buf[cur];
  f.cidx = idx_buf[cur];
  f.in_len = int(len);
  f.k = k;
  f.nchunks = 1;
  f.out_idx = idx;
  launch_select<true, true>(f, int(len), R, 1, stream);
  return hipGetLastError();
}

}  // namespace csa
