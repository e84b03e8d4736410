// Top-k selection of indexer scores.
//
// "DeepSeek-V4-Flash 架构：一个 token 的旅程", section "少读 KV 之前，Indexer
// 仍要给历史打分" (top-k fixes what the main attention reads) and "LLM Atlas:
// DeepSeek" §19 (k = 512 for Flash, 1024 for Pro).
//
// Scores map to order-preserving 32-bit keys (invisible / -inf -> 0).  A
// workgroup stages up to M keys of one row in LDS and finds the exact k-th
// largest key with few barriers: a histogram over 256 equal-width score bins
// (built straight from registers into per-wave LDS histograms) locates the
// bin of the k-th score, one wave scans the bins, the keys of that bin are
// gathered into a short list and ranked against each other, which yields
// the exact threshold key (8-bit radix passes over the bin remain as the
// fallback for heavily tied data).  The kept set is then written by an
// ordered compaction: every thread owns a contiguous run of positions, one
// block scan of packed (greater, equal) counts gives each thread its output
// offset and its share of the threshold-equal keys, so ties go to the lowest
// index and the output is sorted by index -- deterministic run to run.
//
// Rows longer than one LDS tile are cut into chunks; each chunk keeps its own
// top-k as (key, index) candidates, whose union provably holds the row's
// top-k under the same (key desc, index asc) order.  Candidate lists are
// reduced again until one tile remains.
#include <algorithm>
#include <mutex>

#include "common.h"
#include "kernels.h"

// Scratch of the no-allocation top-k (csa_topk_noalloc): the two chunk
// candidate buffers of rows longer than one tile, for callers that cannot
// allocate.  Every device the library runs on holds its own copy until the
// process ends.  In host code this name is only a stand-in for the device
// array: host code uses the address that topk_scratch() looks up.
static __device__ __align__(256) unsigned char scratch[CSA_TOPK_NOALLOC_SCRATCH_BYTES];

namespace csa {
namespace {

constexpr int kMaxTile = 16384;

__device__ __forceinline__ uint32_t score_key(float f) {
  if (f == -INFINITY) return 0u;
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Score value of a valid key (inverse of score_key).
__device__ __forceinline__ float key_value(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
}

// Exclusive scan over the block; returns the exclusive prefix, *total the sum.
template <int THREADS>
__device__ __forceinline__ uint32_t block_scan(uint32_t v, uint32_t* wsum, uint32_t* total) {
  constexpr int W = THREADS / kWave;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const uint32_t x = wave_incl_scan(v);
  if (lane == kWave - 1) wsum[wave] = x;
  __syncthreads();
  // every thread adds up the (at most 16) wave totals itself: LDS broadcasts
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < W; ++i) {
    const uint32_t t = wsum[i];
    before += i < wave ? t : 0u;
    all += t;
  }
  *total = all;
  __syncthreads();  // wsum may be reused by the next scan
  return before + x - v;
}

struct SelectArgs {
  const float* scores;    // raw source: [R, N]
  const int* n_valid;     // raw source: [R] or null
  const uint32_t* ckey;   // candidate source: [R, in_len]
  const int* cidx;
  int in_len;             // raw: N; candidates: entries per row
  int k;
  int nchunks;            // chunks per row at this level (output stride)
  int vec4;               // raw source: N % 4 == 0 and 16-byte aligned rows
  int* out_idx;           // final: [R, k]
  uint32_t* okey;         // chunked: [R, nchunks*k]
  int* oidx;
};

// LDS position of staged key i: 16-byte chunk i/4 moves to chunk
// (i/4) ^ ((i/64) % 16).  A thread's run of 16 keys (four chunks 64 bytes
// apart from its neighbours') then spreads over all bank groups when read as
// 16-byte vectors, and the coalesced writes of 64 consecutive keys stay a
// permutation of 16 consecutive chunks.
__device__ __forceinline__ int lds_swizzle(int i) { return (((i >> 2) ^ ((i >> 6) & 15)) << 2) | (i & 3); }

template <int THREADS, int ITEMS, bool FROM_CAND, bool FINAL>
__global__ __launch_bounds__(THREADS) void topk_select(SelectArgs a) {
  constexpr int M = THREADS * ITEMS;
  static_assert(ITEMS % 4 == 0, "keys move in 16-byte groups");
  constexpr int W = THREADS / kWave;
  __shared__ __attribute__((aligned(16))) uint32_t keys[M];
  __shared__ __attribute__((aligned(16))) int idxs[FROM_CAND ? M : 1];
  __shared__ uint32_t hist[W][256];  // one histogram per wave: no cross-wave atomic contention
  __shared__ uint32_t wsum[W + 1];
  __shared__ uint32_t wcount[W];
  __shared__ float wlo[W], whi[W];
  __shared__ __attribute__((aligned(16))) uint32_t list[THREADS];  // keys of the threshold bin, then zeros
  __shared__ uint32_t nlist, sh_bin, sh_above, sh_thr, sh_need;
  __shared__ uint32_t pick[2];

  const int row = blockIdx.x, chunk = blockIdx.y, tid = threadIdx.x;
  const int lane = tid % kWave, wave = tid / kWave;
  const int64_t base = int64_t(chunk) * M;
  int len = a.in_len;
  if (!FROM_CAND && a.n_valid != nullptr) len = min(len, max(a.n_valid[row], 0));
  for (int i = lane; i < 256; i += kWave) hist[wave][i] = 0;  // own wave's histogram
  if (tid == 0) nlist = 0;
  list[tid] = 0u;  // a zero key is never larger than, nor equal to, a valid key

  // Coalesced, straight-line loads (position tid + t*THREADS, or four keys
  // at 4*(tid + j*THREADS) when rows are 16-byte aligned); the keys then
  // pass once through LDS so that every thread owns the contiguous run
  // [tid*ITEMS, tid*ITEMS + ITEMS) in registers for the rest of the kernel.
  {
    uint32_t kin[ITEMS];
    int iin[FROM_CAND ? ITEMS : 1];
    const int64_t rbase = int64_t(row) * a.in_len;
    if (a.vec4 && base < len) {
      // four keys per load: position 4*(tid + j*THREADS) + c; the last
      // quad of the row bounds the address, the length masks the keys
      const int64_t last4 = a.in_len - 4;
#pragma unroll
      for (int j = 0; j < ITEMS / 4; ++j) {
        const int64_t p = base + 4 * (tid + j * THREADS);
        const int64_t q = rbase + (p < last4 ? p : last4);
        uint4 v;
        if constexpr (FROM_CAND) {
          v = *reinterpret_cast<const uint4*>(a.ckey + q);
          const int4 w = *reinterpret_cast<const int4*>(a.cidx + q);
          iin[4 * j] = w.x; iin[4 * j + 1] = w.y; iin[4 * j + 2] = w.z; iin[4 * j + 3] = w.w;
        } else {
          v = *reinterpret_cast<const uint4*>(a.scores + q);
        }
        kin[4 * j] = v.x; kin[4 * j + 1] = v.y; kin[4 * j + 2] = v.z; kin[4 * j + 3] = v.w;
      }
#pragma unroll
      for (int t = 0; t < ITEMS; ++t) {
        const bool in = base + 4 * (tid + (t / 4) * THREADS) + t % 4 < len;
        if constexpr (FROM_CAND) kin[t] = in ? kin[t] : 0u;
        else kin[t] = in ? score_key(__uint_as_float(kin[t])) : 0u;
      }
    } else if (base < len) {
      const int64_t last = len - 1;
#pragma unroll
      for (int t = 0; t < ITEMS; ++t) {
        const int64_t p = base + tid + t * THREADS;
        const int64_t q = p < last ? p : last;
        if constexpr (FROM_CAND) {
          kin[t] = a.ckey[rbase + q];
          iin[t] = a.cidx[rbase + q];
        } else {
          kin[t] = __float_as_uint(a.scores[rbase + q]);
        }
      }
#pragma unroll
      for (int t = 0; t < ITEMS; ++t) {
        const bool in = base + tid + t * THREADS < len;
        if constexpr (FROM_CAND) kin[t] = in ? kin[t] : 0u;
        else kin[t] = in ? score_key(__uint_as_float(kin[t])) : 0u;
      }
    } else {
#pragma unroll
      for (int t = 0; t < ITEMS; ++t) {
        kin[t] = 0u;
        if constexpr (FROM_CAND) iin[t] = -1;
      }
    }
    // count and score range of the valid keys, straight from the loads (the
    // staging barrier below publishes them with the keys)
    {
      uint32_t ok = 0;
      float lo = INFINITY, hi = -INFINITY;
#pragma unroll
      for (int t = 0; t < ITEMS; ++t) {
        if (kin[t] != 0u) {
          const float f = key_value(kin[t]);
          ++ok;
          lo = fminf(lo, f);
          hi = fmaxf(hi, f);
        }
      }
      ok = wave_sum_u32(ok);
      lo = wave_min(lo);
      hi = wave_max(hi);
      if (lane == 0) { wcount[wave] = ok; wlo[wave] = lo; whi[wave] = hi; }
    }
    if (a.vec4) {
#pragma unroll
      for (int j = 0; j < ITEMS / 4; ++j) {
        const int at = lds_swizzle(4 * (tid + j * THREADS));
        *reinterpret_cast<uint4*>(&keys[at]) = uint4{kin[4 * j], kin[4 * j + 1], kin[4 * j + 2], kin[4 * j + 3]};
        if constexpr (FROM_CAND)
          *reinterpret_cast<int4*>(&idxs[at]) = int4{iin[4 * j], iin[4 * j + 1], iin[4 * j + 2], iin[4 * j + 3]};
      }
    } else {
#pragma unroll
      for (int t = 0; t < ITEMS; ++t) {
        keys[lds_swizzle(tid + t * THREADS)] = kin[t];
        if constexpr (FROM_CAND) idxs[lds_swizzle(tid + t * THREADS)] = iin[t];
      }
    }
  }
  __syncthreads();
  uint32_t key[ITEMS];
  int kidx[FROM_CAND ? ITEMS : 1];
#pragma unroll
  for (int t = 0; t < ITEMS; t += 4) {
    const uint4 v = *reinterpret_cast<const uint4*>(&keys[lds_swizzle(tid * ITEMS + t)]);
    key[t] = v.x; key[t + 1] = v.y; key[t + 2] = v.z; key[t + 3] = v.w;
    if constexpr (FROM_CAND) {
      const int4 w = *reinterpret_cast<const int4*>(&idxs[lds_swizzle(tid * ITEMS + t)]);
      kidx[t] = w.x; kidx[t + 1] = w.y; kidx[t + 2] = w.z; kidx[t + 3] = w.w;
    }
  }
  uint32_t n_ok = 0;
  float lo = INFINITY, hi = -INFINITY;  // score range of the valid keys
#pragma unroll
  for (int w = 0; w < W; ++w) { n_ok += wcount[w]; lo = fminf(lo, wlo[w]); hi = fmaxf(hi, whi[w]); }

  uint32_t thr = 0, need_eq = 0;
  if (n_ok > uint32_t(a.k)) {
    // 256 equal-width bins of the score value between the smallest and the
    // largest score: a monotone function of the score, so higher bins hold
    // larger keys, and the bins spread the scores out (the top key bits --
    // sign and exponent -- do not).
    const float inv = hi > lo ? 256.f / (hi - lo) : 0.f;
    auto bin = [&](uint32_t key) -> uint32_t {
      const uint32_t x = uint32_t((key_value(key) - lo) * inv);
      return x < 255u ? x : 255u;
    };
    // each item's bin, kept (packed bytes) for the gather and the radix passes
    uint32_t binp[(ITEMS + 3) / 4] = {};
#pragma unroll
    for (int t = 0; t < ITEMS; ++t) {
      if (key[t] != 0u) {
        const uint32_t bt = bin(key[t]);
        binp[t / 4] |= bt << (8 * (t % 4));
        atomicAdd(&hist[wave][bt], 1u);
      }
    }
    auto bin_of = [&](int t) { return (binp[t / 4] >> (8 * (t % 4))) & 255u; };
    __syncthreads();
    // one wave scans the bins from the top: lane L covers bins 255-4L .. 252-4L
    if (wave == 0) {
      uint32_t cnt[4], own = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        cnt[j] = 0;
#pragma unroll
        for (int w = 0; w < W; ++w) cnt[j] += hist[w][255 - 4 * lane - j];
        own += cnt[j];
      }
      const uint32_t incl = wave_incl_scan(own);
      uint32_t above = incl - own;  // keys in bins above this lane's
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (above < uint32_t(a.k) && above + cnt[j] >= uint32_t(a.k)) { sh_bin = 255 - 4 * lane - j; sh_above = above; }
        above += cnt[j];
      }
    }
    __syncthreads();
    const uint32_t sel_bin = sh_bin;
    uint32_t remaining = a.k - sh_above;  // how many keys of that bin are kept
    // one LDS atomic per wave and item slot: lanes take consecutive places
#pragma unroll
    for (int t = 0; t < ITEMS; ++t) {
      const bool m = key[t] != 0u && bin_of(t) == sel_bin;
      const uint64_t bal = __ballot(m);
      if (bal != 0) {
        uint32_t at0 = 0;
        if (lane == 0) at0 = atomicAdd(&nlist, uint32_t(__popcll(bal)));
        at0 = __builtin_amdgcn_readfirstlane(at0);
        const uint32_t at = at0 + uint32_t(__builtin_amdgcn_mbcnt_hi(uint32_t(bal >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(bal), 0)));
        if (m && at < THREADS) list[at] = key[t];
      }
    }
    __syncthreads();
    const uint32_t n = nlist;
    if (n <= THREADS) {
      // rank every key of the bin against the others: the threshold key has
      // fewer than `remaining` larger keys and at least `remaining` >= keys
      if (tid < int(n)) {
        const uint32_t key = list[tid];
        uint32_t gt = 0, eqc = 0;
        // four keys per LDS read (the zeros past the list count for nothing)
        const uint4* l4 = reinterpret_cast<const uint4*>(list);
#pragma unroll 2
        for (uint32_t j = 0; j < n; j += 4) {
          const uint4 v = l4[j / 4];
          gt += uint32_t(v.x > key) + uint32_t(v.y > key) + uint32_t(v.z > key) + uint32_t(v.w > key);
          eqc += uint32_t(v.x == key) + uint32_t(v.y == key) + uint32_t(v.z == key) + uint32_t(v.w == key);
        }
        if (gt < remaining && remaining <= gt + eqc) { sh_thr = key; sh_need = remaining - gt; }
      }
      __syncthreads();
      thr = sh_thr;
      need_eq = sh_need;
    } else {
      // many equal or nearly equal scores: exact 8-bit radix passes over the bin
      uint32_t prefix = 0, mask = 0;
      for (int shift = 24; shift >= 0; shift -= 8) {
        for (int i = tid; i < W * 256; i += THREADS) (&hist[0][0])[i] = 0;
        __syncthreads();
#pragma unroll
        for (int t = 0; t < ITEMS; ++t) {
          const uint32_t kk = key[t];
          if (kk != 0u && (kk & mask) == prefix && bin_of(t) == sel_bin)
            atomicAdd(&hist[wave][(kk >> shift) & 255u], 1u);
        }
        __syncthreads();
        uint32_t hv = 0;
        if (tid < 256) {
#pragma unroll
          for (int w = 0; w < W; ++w) hv += hist[w][255 - tid];
        }
        uint32_t tot;
        const uint32_t ex = block_scan<THREADS>(hv, wsum, &tot);
        if (tid < 256 && ex + hv >= remaining && ex < remaining) { pick[0] = uint32_t(255 - tid); pick[1] = ex; }
        __syncthreads();
        remaining -= pick[1];
        prefix |= pick[0] << shift;
        mask |= 0xffu << shift;
        __syncthreads();
      }
      thr = prefix;
      need_eq = remaining;
    }
  }

  // Ordered compaction over contiguous runs of ITEMS positions.  One scan of
  // packed (greater, equal) counts gives each thread its output offset: the
  // equal keys before it that are kept number min(prefix_eq, need_eq).
  const int j0 = tid * ITEMS;
  uint32_t gt = 0, eq = 0;
#pragma unroll
  for (int t = 0; t < ITEMS; ++t) {
    gt += key[t] > thr;
    eq += (key[t] == thr) && (key[t] != 0u);
  }
  uint32_t tot;
  const uint32_t ex = block_scan<THREADS>((gt << 16) | eq, wsum, &tot);
  const uint32_t p_gt = ex >> 16, p_eq = ex & 0xffffu;
  uint32_t o = p_gt + min(p_eq, need_eq);
  const uint32_t take = need_eq > p_eq ? min(need_eq - p_eq, eq) : 0u;
  const uint32_t n_sel = (tot >> 16) + min(tot & 0xffffu, need_eq);
  uint32_t taken = 0;
  const int64_t obase = FINAL ? int64_t(row) * a.k : (int64_t(row) * a.nchunks + chunk) * a.k;
#pragma unroll
  for (int t = 0; t < ITEMS; ++t) {
    const uint32_t kk = key[t];
    bool sel = kk > thr;
    if (!sel && kk == thr && kk != 0u && taken < take) { sel = true; ++taken; }
    if (sel) {
      int index;
      if constexpr (FROM_CAND) index = kidx[t];
      else index = int(base + j0 + t);
      if constexpr (FINAL) {
        a.out_idx[obase + o] = index;
      } else {
        a.okey[obase + o] = kk;
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

// Launch one selection level.  `tile` is the number of positions one
// workgroup stages (THREADS*ITEMS of the chosen instance).
template <bool FROM_CAND, bool FINAL>
void launch_select(const SelectArgs& a, int tile, int R, int nchunks, hipStream_t s) {
  const dim3 grid(R, nchunks);
  if (tile == 2048)
    hipLaunchKernelGGL((topk_select<256, 8, FROM_CAND, FINAL>), grid, dim3(256), 0, s, a);
  else if (tile == 8192)
    hipLaunchKernelGGL((topk_select<512, 16, FROM_CAND, FINAL>), grid, dim3(512), 0, s, a);
  else
    hipLaunchKernelGGL((topk_select<1024, 16, FROM_CAND, FINAL>), grid, dim3(1024), 0, s, a);
}

int tile_for(int64_t len) { return len <= 2048 ? 2048 : (len <= 8192 ? 8192 : kMaxTile); }

// Levels: rows longer than one tile are first cut into 8192-position chunks
// (512-thread workgroups, several per CU: measured faster than one
// 1024-thread workgroup per 16384 positions); the following levels reduce
// candidate lists in kMaxTile chunks; the last one selects from at most
// kMaxTile positions.
struct Levels {
  int n;
  int64_t len[8];    // positions per row entering level i
  int tile[8];       // positions per workgroup at level i
  int64_t cand_max;  // largest candidate list per row
};

Levels levels_of(int R, int N, int k) {
  Levels L{};
  int64_t len = N;
  const int first = N > kMaxTile ? 8192 : kMaxTile;
  while (true) {
    const int tile = L.n == 0 ? (len > first ? first : tile_for(len)) : (len > kMaxTile ? kMaxTile : tile_for(len));
    L.len[L.n] = len;
    L.tile[L.n] = tile;
    ++L.n;
    if (len <= tile) break;
    len = (len + tile - 1) / tile * k;
    L.cand_max = std::max(L.cand_max, len);
  }
  return L;
}

}  // namespace

TopkPlan plan_topk(int R, int N, int k) {
  const Levels L = levels_of(R, N, k);
  TopkPlan p{L.n - 1, int64_t(R) * L.cand_max, 0};
  p.ws_bytes = p.levels ? size_t(2) * size_t(p.cand_elems) * (sizeof(uint32_t) + sizeof(int)) : 0;
  return p;
}

// Device address of this device's scratch array, looked up once per device
// (with that device current) and kept.
hipError_t topk_scratch(void** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}

hipError_t launch_topk(const float* scores, const int* n_valid, int R, int N, int k, int* idx, void* ws,
                       hipStream_t stream) {
  if (R == 0) return hipSuccess;
  const Levels L = levels_of(R, N, k);
  const TopkPlan plan = plan_topk(R, N, k);
  uint32_t* key_buf[2] = {nullptr, nullptr};
  int* idx_buf[2] = {nullptr, nullptr};
  if (plan.levels) {
    char* w = static_cast<char*>(ws);
    for (int i = 0; i < 2; ++i) {
      key_buf[i] = reinterpret_cast<uint32_t*>(w);
      w += plan.cand_elems * sizeof(uint32_t);
      idx_buf[i] = reinterpret_cast<int*>(w);
      w += plan.cand_elems * sizeof(int);
    }
  }
  int cur = -1;  // -1: the raw score rows
  for (int l = 0; l < L.n; ++l) {
    const bool last = l == L.n - 1;
    const int64_t len = L.len[l];
    const int tile = L.tile[l];
    const int nch = last ? 1 : int((len + tile - 1) / tile);
    SelectArgs a{};
    a.k = k;
    a.in_len = int(len);
    a.nchunks = nch;
    if (cur < 0) {
      a.scores = scores;
      a.n_valid = n_valid;
      a.vec4 = N % 4 == 0 && reinterpret_cast<uintptr_t>(scores) % 16 == 0;
    } else {
      a.ckey = key_buf[cur];
      a.cidx = idx_buf[cur];
      a.vec4 = len % 4 == 0 && reinterpret_cast<uintptr_t>(a.ckey) % 16 == 0 &&
               reinterpret_cast<uintptr_t>(a.cidx) % 16 == 0;
    }
    if (last) {
      a.out_idx = idx;
      if (cur < 0) launch_select<false, true>(a, tile, R, 1, stream);
      else launch_select<true, true>(a, tile, R, 1, stream);
    } else {
      const int nxt = cur < 0 ? 0 : cur ^ 1;
      a.okey = key_buf[nxt];
      a.oidx = idx_buf[nxt];
      if (cur < 0) launch_select<false, false>(a, tile, R, nch, stream);
      else launch_select<true, false>(a, tile, R, nch, stream);
      cur = nxt;
    }
  }
  return hipGetLastError();
}

}  // namespace csa
