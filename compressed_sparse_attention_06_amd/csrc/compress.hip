// Compressor: per-channel softmax pooling of a token group, RMSNorm, RoPE.
//
// "DeepSeek-V4-Flash 架构：一个 token 的旅程", sections "压缩是逐通道的
// learned pooling", "一个通道，逐项算出压缩结果" and "压缩条目必须等整组完成后才可见".
//
// The work is a streaming reduction over the candidate rows of each entry.
// The fast path gives every lane 2, 4 or 8 consecutive channels, so a
// candidate row is one coalesced read per wave, and lays a block's waves out
// over channel groups and candidate groups; the softmax over candidates runs
// on register batches of rows (batch maximum, then one exponential per
// element).  A block with one candidate group finishes its entry in
// registers; several groups merge in LDS.  Few entries with long candidate
// lists are sliced over workgroups that merge through a workspace.  Widths
// that are not a multiple of 128 take a one-wave-per-entry path.
#include <algorithm>

#include "common.h"
#include "kernels.h"
#include "kv4.h"

namespace csa {
namespace {

constexpr int kMaxWavesPerEntry = 16;
// Waves per block by channels per lane: wide lanes hold more registers.
__host__ __device__ constexpr int max_waves(int cpl) { return cpl == 2 ? kMaxWavesPerEntry : 4; }
constexpr int kMaxSplits = 16;
constexpr int kMaxJobs = 4;

// Jobs of one launch: blocks [first[j], first[j+1]) build job j's entries,
// with job j's own plan (its waves per block may be fewer than the launch's:
// the others idle through the barriers).
struct CompressBatch {
  CompressArgs job[kMaxJobs];
  int first[kMaxJobs + 1];
  int gc[kMaxJobs], gr[kMaxJobs], nsplit[kMaxJobs];
  int n;
};

// Split-entry workspace: one arrival counter per entry slot in a fixed block
// of kSplitMaxEntries counters at offset 0, then the partial states (max,
// sum, weighted sum) per channel, slice and entry.  The counters sit at the
// same place whatever the call's entry count, width or ratio, so a
// workspace kept across calls of different shapes always finds them zero.
constexpr int kSplitMaxEntries = 256;
constexpr size_t kSplitCounterBytes = kSplitMaxEntries * sizeof(unsigned);
__host__ __device__ inline size_t split_ws_bytes(int64_t entries, int nsplit, int D) {
  return kSplitCounterBytes + size_t(entries) * nsplit * 3 * D * sizeof(float);
}

struct Task {
  int b;
  int e;
  bool live;
};

__device__ __forceinline__ Task compress_task(const CompressArgs& a, int w) {
  Task t{0, 0, false};
  if (a.pos == nullptr) {
    if (w >= a.B * a.n_entries) return t;
    t.b = w / a.n_entries;
    t.e = a.e0 + w % a.n_entries;
    t.live = a.pt.pages == nullptr || paged_row(a.pt, t.b, t.e) >= 0;
  } else {
    if (w >= a.B) return t;
    const int p = a.pos[w];
    t.b = w;
    if (p < 0 || (p + 1) % a.ratio != 0) return t;
    t.e = p / a.ratio;
    t.live = t.e < a.out_cap && (a.pt.pages == nullptr || paged_row(a.pt, t.b, t.e) >= 0);
  }
  return t;
}

// Quantised output: entry e of sequence b at out + b*out_bstride bytes + e
// rows of kv4_row_bytes (contiguous), or its pool row (paged).
__device__ __forceinline__ unsigned char* kv4_out_row(const CompressArgs& a, int b, int e) {
  const int rb = kv4_row_bytes(a.D, a.rope_dim);
  if (a.pt.pages) return static_cast<unsigned char*>(a.out) + paged_row(a.pt, b, e) * rb;
  return static_cast<unsigned char*>(a.out) + int64_t(b) * a.out_bstride + int64_t(e) * rb;
}

// Row of token `tok` inside a sequence's span (span mode) or ring (ring mode).
__device__ __forceinline__ int64_t token_row(const CompressArgs& a, int64_t tok) {
  return a.pos == nullptr ? tok - a.tok0 : tok % a.T;
}

// Fast path: D = 64*CPL*gc.  Lane l of a wave owns channels CPL*l ..
// CPL*l + CPL-1 of a (64*CPL)-channel group, so one candidate row is one
// coalesced read per wave.  The block's gc*gr waves tile (channel group) x
// (candidate group): a wave runs the softmax over its share of the
// candidates for its channels, in batches of rows held in registers (the
// batch maximum first, then one exponential per element; the next batch is
// in flight meanwhile).  With one candidate group the wave's registers hold
// the pooled values; otherwise the per-wave (max, sum, weighted sum) states
// meet in LDS and every thread of the block merges channels.  The RMS
// statistic is one block reduction; the RoPE pairs of the trailing slice are
// rotated with a table built while the first rows were in flight.
// blockIdx.x is (job, entry) of the batch, blockIdx.y the candidate slice of
// a split entry (split entries always take channel pairs, one group).
template <int CPL, bool BF16>
__global__ __launch_bounds__(kWave* max_waves(CPL)) void compress_lanes(CompressBatch batch) {
  extern __shared__ float lds[];  // states [gr][3][D] | y [D] | RoPE (cos, sin) [rope_dim] | partial sums [16]
  // the wave index is uniform: the candidate and row arithmetic stays scalar
  const int lane = threadIdx.x % kWave, wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int nthr = blockDim.x;
  int job = 0;
  for (int k = 1; k < batch.n; ++k)
    if (int(blockIdx.x) >= batch.first[k]) job = k;
  const CompressArgs a = batch.job[job];
  const int gc = batch.gc[job], gr = batch.gr[job], nsplit = batch.nsplit[job];
  const int w = int(blockIdx.x) - batch.first[job];             // entry task within the job
  const int entries = batch.first[job + 1] - batch.first[job];  // the job's entry tasks
  if (int(blockIdx.y) >= nsplit) return;
  const bool active = wave < gc * gr;  // else an idle wave of a smaller job
  const Task task = compress_task(a, w);
  if (!task.live) return;
  const int D = a.D, r = a.ratio, e = task.e;
  float* st = lds;
  float* ybuf = lds + size_t(gr) * 3 * D;
  float* rope_tab = ybuf + D;
  float* red = rope_tab + a.rope_dim;
  const int cg = wave % gc, rg = wave / gc;
  const int c0 = cg * kWave * CPL + lane * CPL;
  const int64_t seq = int64_t(task.b) * a.in_bstride;

  // candidate c: previous-group token (e-1)*r + c for c < cp, else current token
  const int cp = (a.overlap && e > 0) ? r : 0;
  const int C = cp + r;
  // blockIdx.y takes one slice of the candidates; the waves share it out
  const int cps = (C + nsplit - 1) / nsplit;
  const int blo = min(C, int(blockIdx.y) * cps), bhi = min(C, blo + cps);
  const int per = (bhi - blo + gr - 1) / gr;
  const int cb = min(bhi, blo + rg * per), ce = min(bhi, cb + per);
  // candidates are consecutive tokens from t_first; their rows follow one
  // another in the span, or wrap once around the ring (C <= 2r <= T)
  const int64_t t_first = int64_t(e) * r - cp;
  const int64_t row_first = a.pos == nullptr ? t_first - a.tok0 : t_first % a.T;

  // rows stay in their storage format until absorbed: bf16 pairs or fp32 bits
  constexpr int RW = BF16 ? CPL / 2 : CPL;
  constexpr int kBatch = (BF16 ? 32 : 16) / CPL;
  uint32_t g0[kBatch][RW], v0[kBatch][RW], g1[kBatch][RW], v1[kBatch][RW];
  // a row's address is a scalar base (uniform) plus the lane's byte offset
  constexpr int kEs = BF16 ? 2 : 4;
  const uint32_t lane_b = uint32_t(c0) * kEs;
  auto load_raw = [](const char* p, uint32_t (&w)[RW]) {
    if constexpr (RW == 8) {
      const uint4 x = reinterpret_cast<const uint4*>(p)[0], y = reinterpret_cast<const uint4*>(p)[1];
      w[0] = x.x; w[1] = x.y; w[2] = x.z; w[3] = x.w; w[4] = y.x; w[5] = y.y; w[6] = y.z; w[7] = y.w;
    } else if constexpr (RW == 4) {
      const uint4 x = *reinterpret_cast<const uint4*>(p);
      w[0] = x.x; w[1] = x.y; w[2] = x.z; w[3] = x.w;
    } else if constexpr (RW == 2) {
      const uint2 x = *reinterpret_cast<const uint2*>(p);
      w[0] = x.x; w[1] = x.y;
    } else {
      w[0] = *reinterpret_cast<const uint32_t*>(p);
    }
  };
  auto load_batch = [&](int c, uint32_t (&g)[kBatch][RW], uint32_t (&v)[kBatch][RW]) {
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      if (c + j < ce) {
        const int cc = c + j;
        const bool prev = cc < cp;
        int64_t row = row_first + cc;
        if (a.pos != nullptr && row >= a.T) row -= a.T;
        const int64_t off = (seq + row * D) * kEs;
        const char* gp = static_cast<const char*>(prev ? a.gate_prev : a.gate) + off;
        const char* vp = static_cast<const char*>(prev ? a.kv_prev : a.kv) + off;
        load_raw(gp + lane_b, g[j]);
        load_raw(vp + lane_b, v[j]);
      }
    }
  };
  auto elem = [&](const uint32_t (&w)[RW], int i) -> float {
    if constexpr (BF16) return (i & 1) ? bf16_hi(w[i / 2]) : bf16_lo(w[i / 2]);
    else return __uint_as_float(w[i]);
  };
  if (cb < ce) load_batch(cb, g0, v0);
  // a one-group entry's RMSNorm gains travel with its first rows (read in
  // the epilogue they would be one more round trip after the merge)
  float gam[CPL];
  if (gr == 1 && active) {
#pragma unroll
    for (int i = 0; i < CPL; ++i) gam[i] = a.gamma[c0 + i];
  }

  // RoPE table while the first rows are in flight
  const int rope0 = D - a.rope_dim;
  for (int i = threadIdx.x; i < a.rope_dim / 2; i += nthr)
    rope_cos_sin(int64_t(e) * r, i, a.rope_dim, a.rope_log2_base, &rope_tab[2 * i], &rope_tab[2 * i + 1]);

  // running state per channel, the maximum kept in the log2 domain
  float m[CPL], s[CPL], acc[CPL];
#pragma unroll
  for (int i = 0; i < CPL; ++i) { m[i] = -INFINITY; s[i] = 0.f; acc[i] = 0.f; }
  auto absorb = [&](int c, const uint32_t (&g)[kBatch][RW], const uint32_t (&v)[kBatch][RW]) {
    float gf[kBatch][CPL];
    float mb[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) mb[i] = -INFINITY;
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        gf[j][i] = elem(g[j], i);
        if (c + j < ce) mb[i] = fmaxf(mb[i], gf[j][i]);
      }
    }
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const float mn = fmaxf(m[i], mb[i] * kLog2e);
      const float keep = fast_exp2(m[i] - mn);  // 0 while nothing was absorbed
      s[i] *= keep;
      acc[i] *= keep;
      m[i] = mn;
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      if (c + j < ce) {
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
          const float pj = fast_exp2(fmaf(gf[j][i], kLog2e, -m[i]));
          s[i] += pj;
          acc[i] = fmaf(pj, elem(v[j], i), acc[i]);
        }
      }
    }
  };
  for (int c = cb; c < ce; c += 2 * kBatch) {
    if (c + kBatch < ce) load_batch(c + kBatch, g1, v1);
    absorb(c, g0, v0);
    if (c + kBatch < ce) {
      if (c + 2 * kBatch < ce) load_batch(c + 2 * kBatch, g0, v0);
      absorb(c + kBatch, g1, v1);
    }
  }
  // y: the pooled value of each of the lane's own channels, when the block
  // has one candidate group (else the block's pooled row goes to LDS)
  float y[CPL];
  float ss = 0.f;
  if (nsplit == 1 && gr == 1) {
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      y[i] = active ? acc[i] / s[i] : 0.f;
      ss = fmaf(y[i], y[i], ss);
    }
  } else if (nsplit == 1) {
    if (active) {
      float* mine = st + size_t(rg) * 3 * D + c0;
#pragma unroll
      for (int i = 0; i < CPL; i += 2) {
        *reinterpret_cast<float2*>(mine + i) = float2{m[i], m[i + 1]};
        *reinterpret_cast<float2*>(mine + D + i) = float2{s[i], s[i + 1]};
        *reinterpret_cast<float2*>(mine + 2 * D + i) = float2{acc[i], acc[i + 1]};
      }
    }
    __syncthreads();
    // merge the candidate groups channel by channel
    for (int c = threadIdx.x; c < D; c += nthr) {
      float mx = -INFINITY;
      for (int g = 0; g < gr; ++g) mx = fmaxf(mx, st[size_t(g) * 3 * D + c]);
      float S = 0.f, A = 0.f;
      for (int g = 0; g < gr; ++g) {
        const float* o = st + size_t(g) * 3 * D + c;
        if (o[0] == -INFINITY) continue;  // that group had no candidate
        const float f = fast_exp2(o[0] - mx);
        S = fmaf(o[D], f, S);
        A = fmaf(o[2 * D], f, A);
      }
      const float yc = A / S;
      ybuf[c] = yc;
      ss = fmaf(yc, yc, ss);
    }
  } else if constexpr (CPL == 2) {
    // Split entry (one candidate group, a channel pair per lane): publish
    // this slice's states; the block that arrives last (one counter per
    // entry) merges every slice and finishes the entry.  Nothing waits on
    // another block.  The states travel as device-scope stores and loads,
    // which write through and read past the caches that are private to a
    // group of compute units; a wave's stores have reached that level once
    // its store counter drains, and the barrier orders every wave's drain
    // before thread 0's arrival.  No device-scope fence is needed (here one
    // would write back or invalidate a whole L2).
    unsigned* ctr = static_cast<unsigned*>(a.ws);
    float* part = reinterpret_cast<float*>(static_cast<char*>(a.ws) + kSplitCounterBytes) + size_t(w) * nsplit * 3 * D;
    // one 64-bit device-scope store per state and lane: the lane's channel pair
    auto st2 = [](float* p, float x0, float x1) {
      const uint64_t v = uint64_t(__float_as_uint(x0)) | (uint64_t(__float_as_uint(x1)) << 32);
      __hip_atomic_store(reinterpret_cast<uint64_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    float* pp = part + size_t(blockIdx.y) * 3 * D + c0;
    st2(pp, m[0], m[1]);
    st2(pp + D, s[0], s[1]);
    st2(pp + 2 * D, acc[0], acc[1]);
    __shared__ bool last;
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's states are out
    __syncthreads();
    if (threadIdx.x == 0)
      last = __hip_atomic_fetch_add(&ctr[w], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
             unsigned(nsplit - 1);
    __syncthreads();
    if (!last) return;
    // every lane merges its own channel pair over the slices, all loads at once
    auto ld2 = [](const float* p) {
      return __hip_atomic_load(reinterpret_cast<const uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    uint64_t pm[kMaxSplits], ps[kMaxSplits], pa[kMaxSplits];
#pragma unroll
    for (int k = 0; k < kMaxSplits; ++k) {
      if (k < nsplit) {
        const float* q = part + size_t(k) * 3 * D + c0;
        pm[k] = ld2(q);
        ps[k] = ld2(q + D);
        pa[k] = ld2(q + 2 * D);
      }
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      auto half = [i](uint64_t v) { return __uint_as_float(uint32_t(v >> (32 * i))); };
      float mx = -INFINITY;
#pragma unroll
      for (int k = 0; k < kMaxSplits; ++k)
        if (k < nsplit) mx = fmaxf(mx, half(pm[k]));
      float S = 0.f, A = 0.f;
#pragma unroll
      for (int k = 0; k < kMaxSplits; ++k) {
        if (k < nsplit && half(pm[k]) != -INFINITY) {  // slices without candidates hold no state
          const float f = fast_exp2(half(pm[k]) - mx);
          S = fmaf(half(ps[k]), f, S);
          A = fmaf(half(pa[k]), f, A);
        }
      }
      y[i] = A / S;
      ss = fmaf(y[i], y[i], ss);
    }
    if (threadIdx.x == 0)  // every slice has arrived: rearm for the next call
      __hip_atomic_store(&ctr[w], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // RMS over the row: one block reduction (its barrier also publishes the
  // RoPE table and the pooled row)
  ss = wave_sum(ss);
  if (lane == 0) red[wave] = ss;
  __syncthreads();
  float tot = 0.f;
  for (int wv = 0; wv < nthr / kWave; ++wv) tot += red[wv];
  const float inv_rms = rsqrtf(tot / float(D) + a.eps);
  const int64_t o = a.pt.pages ? paged_row(a.pt, task.b, e) * D : int64_t(task.b) * a.out_bstride + int64_t(e) * D;

  if (gr == 1) {
    // the lane's own channels, rotated in place (RoPE pairs never straddle
    // lanes) and stored with one vector store
    if (active) {
#pragma unroll
      for (int i = 0; i < CPL; ++i) y[i] *= inv_rms * gam[i];
#pragma unroll
      for (int i = 0; i < CPL; i += 2) {
        const int ch = c0 + i;
        if (ch >= rope0) {
          const float cs = rope_tab[ch - rope0], sn = rope_tab[ch - rope0 + 1];
          const float x0 = y[i], x1 = y[i + 1];
          y[i] = x0 * cs - x1 * sn;
          y[i + 1] = x0 * sn + x1 * cs;
        }
      }
    }
    if (a.out_dtype == CSA_KV4) {  // quantised cache row: staged in LDS, written by wave 0
      if (active) {
#pragma unroll
        for (int i = 0; i < CPL; ++i) ybuf[c0 + i] = y[i];
      }
      __syncthreads();
      if (wave == 0) kv4_store_row(ybuf, D, a.rope_dim, kv4_out_row(a, task.b, e));
      return;
    }
    if (!active) return;
    if (a.out_dtype == CSA_BF16) {
      uint32_t* dst = static_cast<uint32_t*>(a.out) + (o + c0) / 2;
      if constexpr (CPL == 8)
        *reinterpret_cast<uint4*>(dst) = uint4{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]),
                                               pack_bf16x2(y[4], y[5]), pack_bf16x2(y[6], y[7])};
      else if constexpr (CPL == 4)
        *reinterpret_cast<uint2*>(dst) = uint2{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
      else
        *dst = pack_bf16x2(y[0], y[1]);
    } else {
      float* dst = static_cast<float*>(a.out) + o + c0;
#pragma unroll
      for (int i = 0; i < CPL; i += 2) *reinterpret_cast<float2*>(dst + i) = float2{y[i], y[i + 1]};
    }
    return;
  }
  // scale, rotate the trailing pairs, store one pair per thread
  for (int q = threadIdx.x; q < D / 2; q += nthr) {
    const int ch = 2 * q;
    float y0 = ybuf[ch] * inv_rms * a.gamma[ch], y1 = ybuf[ch + 1] * inv_rms * a.gamma[ch + 1];
    if (ch >= rope0) {
      const float cs = rope_tab[ch - rope0], sn = rope_tab[ch - rope0 + 1];
      const float x0 = y0, x1 = y1;
      y0 = x0 * cs - x1 * sn;
      y1 = x0 * sn + x1 * cs;
    }
    if (a.out_dtype == CSA_KV4) {  // in place: this thread alone reads and writes the pair
      ybuf[ch] = y0;
      ybuf[ch + 1] = y1;
    } else if (a.out_dtype == CSA_BF16) {
      static_cast<uint32_t*>(a.out)[(o + ch) / 2] = pack_bf16x2(y0, y1);
    } else {
      *reinterpret_cast<float2*>(static_cast<float*>(a.out) + o + ch) = float2{y0, y1};
    }
  }
  if (a.out_dtype == CSA_KV4) {
    __syncthreads();
    if (wave == 0) kv4_store_row(ybuf, D, a.rope_dim, kv4_out_row(a, task.b, e));
  }
}

// General path: any D (<= 8192), either dtype; one wave per entry, the pooled
// row staged in LDS so that RoPE pairs can straddle lanes.
__global__ __launch_bounds__(kWave) void compress_any(CompressArgs a) {
  extern __shared__ float ybuf[];
  const int lane = threadIdx.x;
  const Task task = compress_task(a, blockIdx.x);
  if (!task.live) return;
  const int D = a.D, r = a.ratio, e = task.e;
  const int64_t seq = int64_t(task.b) * a.in_bstride;
  float ss = 0.f;
  for (int c = lane; c < D; c += kWave) {
    float m = -INFINITY, s = 0.f, acc = 0.f;
    auto absorb = [&](const void* vals, const void* gates, int64_t tok) {
      const int64_t off = seq + token_row(a, tok) * D + c;
      const float gl = load_elem(gates, a.in_dtype, off) * kLog2e;
      const float v = load_elem(vals, a.in_dtype, off);
      const float mn = fmaxf(m, gl);
      const float keep = fast_exp2(m - mn);
      const float pj = fast_exp2(gl - mn);
      s = s * keep + pj;
      acc = acc * keep + pj * v;
      m = mn;
    };
    if (a.overlap && e > 0)
      for (int64_t t = int64_t(e - 1) * r; t < int64_t(e) * r; ++t) absorb(a.kv_prev, a.gate_prev, t);
    for (int64_t t = int64_t(e) * r; t < int64_t(e + 1) * r; ++t) absorb(a.kv, a.gate, t);
    const float y = acc / s;
    ybuf[c] = y;
    ss += y * y;
  }
  ss = wave_sum(ss);
  const float inv_rms = rsqrtf(ss / float(D) + a.eps);
  __syncthreads();
  for (int c = lane; c < D; c += kWave) ybuf[c] *= inv_rms * a.gamma[c];
  __syncthreads();
  const int rope0 = D - a.rope_dim;
  for (int i = lane; i < a.rope_dim / 2; i += kWave) {
    float cs, sn;
    rope_cos_sin(int64_t(e) * r, i, a.rope_dim, a.rope_log2_base, &cs, &sn);
    const float x0 = ybuf[rope0 + 2 * i], x1 = ybuf[rope0 + 2 * i + 1];
    ybuf[rope0 + 2 * i] = x0 * cs - x1 * sn;
    ybuf[rope0 + 2 * i + 1] = x0 * sn + x1 * cs;
  }
  __syncthreads();
  if (a.out_dtype == CSA_KV4) {
    kv4_store_row(ybuf, D, a.rope_dim, kv4_out_row(a, task.b, e));
    return;
  }
  const int64_t o = a.pt.pages ? paged_row(a.pt, task.b, e) * D : int64_t(task.b) * a.out_bstride + int64_t(e) * D;
  for (int c = lane; c < D; c += kWave) store_elem(a.out, a.out_dtype, o + c, ybuf[c]);
}

}  // namespace

CompressPlan plan_compress(int64_t entries, int D, int ratio, int overlap) {
  CompressPlan p{false, 2, 0, 0, 1, 0};
  if (D % 128 != 0) return p;
  // Few entries (decode): a channel pair per lane, so that the block's waves
  // cover the entry's channels and candidates.  Many entries (prefill): as
  // many channels per lane as divide the row, so that one wave reads whole
  // rows with 16-byte loads and keeps more bytes in flight.
  const int wide = D % 512 == 0 ? 8 : (D % 256 == 0 ? 4 : 2);
  p.cpl = (entries >= 512 || D / 128 > kMaxWavesPerEntry) ? wide : 2;
  const int gc = D / (kWave * p.cpl);
  if (gc > max_waves(p.cpl)) return p;
  p.lanes = true;
  p.gc = gc;
  const int64_t cand = int64_t(1 + overlap) * ratio;
  // Long candidate lists of few entries (the heavily compressed role at
  // decode) would leave each entry's rows to one compute unit, whose
  // outstanding reads then bound the time: slice them over blocks, about
  // sixteen rows each (measured against 8 and 32: the last block's merge
  // reads every slice's states).
  if (p.cpl == 2 && cand >= 64 && entries <= kSplitMaxEntries) p.nsplit = int(cand / 16 < kMaxSplits ? cand / 16 : kMaxSplits);
  const int64_t cpb = (cand + p.nsplit - 1) / p.nsplit;
  // candidate groups: at least eight candidates per wave (one register batch;
  // a CSA entry's eight rows stay in one group, which then finishes in
  // registers without the LDS merge -- measured faster than spreading two
  // rows over each of 16 waves); a split entry keeps one group per block,
  // whose waves publish their states straight from registers
  const int per_min = 8;
  int64_t gr = (cpb + per_min - 1) / per_min;
  const int wmax = max_waves(p.cpl) / gc;
  gr = gr < 1 ? 1 : (gr > wmax ? wmax : gr);
  p.gr = p.nsplit > 1 ? 1 : int(gr);
  if (p.nsplit > 1) p.ws_bytes = split_ws_bytes(entries, p.nsplit, D);
  return p;
}

namespace {

int job_tasks(const CompressArgs& a) { return a.pos == nullptr ? a.B * a.n_entries : a.B; }

bool lanes_ready(const CompressArgs& a, const CompressPlan& p) {
  auto al = [](const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15u) == 0; };
  const int in_es = a.in_dtype == CSA_BF16 ? 2 : 4, out_es = a.out_dtype == CSA_BF16 ? 2 : (a.out_dtype == CSA_KV4 ? 1 : 4);
  return p.lanes && al(a.kv) && al(a.gate) && al(a.kv_prev) && al(a.gate_prev) && al(a.out) &&
         (a.in_bstride * in_es) % 16 == 0 && (a.out_bstride * out_es) % 16 == 0;
}

hipError_t launch_lanes(const CompressBatch& b, int cpl, bool bf, int waves, int nsplit, size_t lds,
                        hipStream_t stream) {
  const dim3 grid(b.first[b.n], nsplit), block(kWave * waves);
#define CSA_COMPRESS_CASE(C)                                                                 \
  if (cpl == C) {                                                                            \
    if (bf) hipLaunchKernelGGL((compress_lanes<C, true>), grid, block, lds, stream, b);      \
    else hipLaunchKernelGGL((compress_lanes<C, false>), grid, block, lds, stream, b);        \
  }
  CSA_COMPRESS_CASE(2)
  CSA_COMPRESS_CASE(4)
  CSA_COMPRESS_CASE(8)
#undef CSA_COMPRESS_CASE
  return hipGetLastError();
}

}  // namespace

hipError_t launch_compress(const CompressArgs* jobs, const CompressPlan* plans, int n, hipStream_t stream) {
  // Jobs on the lane kernel with one block per entry and the same lane layout
  // and input dtype share a launch (up to kMaxJobs); the rest run alone.
  bool done[CSA_MAX_COMPRESS_JOBS] = {};
  for (int i = 0; i < n; ++i) {
    if (done[i]) continue;
    done[i] = true;
    const CompressArgs& a = jobs[i];
    const CompressPlan& p = plans[i];
    if (job_tasks(a) == 0) continue;
    if (!lanes_ready(a, p)) {
      hipLaunchKernelGGL(compress_any, dim3(job_tasks(a)), dim3(kWave), a.D * sizeof(float), stream, a);
      const hipError_t err = hipGetLastError();
      if (err != hipSuccess) return err;
      continue;
    }
    CompressBatch b{};
    int waves = 0;
    size_t lds = 0;
    auto add = [&](const CompressArgs& x, const CompressPlan& q) {
      const int k = b.n++;
      b.job[k] = x;
      b.gc[k] = q.gc;
      b.gr[k] = q.gr;
      b.nsplit[k] = q.nsplit;
      b.first[k + 1] = b.first[k] + job_tasks(x);
      waves = std::max(waves, q.gc * q.gr);
      lds = std::max(lds, (size_t(q.gr) * 3 * x.D + x.D + x.rope_dim + kMaxWavesPerEntry) * sizeof(float));
    };
    add(a, p);
    if (p.nsplit == 1) {
      for (int k = i + 1; k < n && b.n < kMaxJobs; ++k) {
        if (done[k] || job_tasks(jobs[k]) == 0 || !lanes_ready(jobs[k], plans[k])) continue;
        if (plans[k].nsplit != 1 || plans[k].cpl != p.cpl || jobs[k].in_dtype != a.in_dtype) continue;
        done[k] = true;
        add(jobs[k], plans[k]);
      }
    }
    const hipError_t err = launch_lanes(b, p.cpl, a.in_dtype == CSA_BF16, waves, p.nsplit, lds, stream);
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace csa
