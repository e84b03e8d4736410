// Compressor: per-channel softmax pooling of a token group, RMSNorm, RoPE.
//
// "DeepSeek-V4-Flash 架构：一个 token 的旅程", sections "压缩是逐通道的
// learned pooling", "一个通道，逐项算出压缩结果" and "压缩条目必须等整组完成后才可见".
//
// The work is a bandwidth-bound streaming reduction.  Each lane owns D/64
// consecutive channels, so every candidate row is one coalesced read of D
// elements by a wave; the softmax over candidates runs online in registers
// (running max, running sum, running weighted sum) with several rows in
// flight; long candidate lists (HCA's 128 rows) are split over up to eight
// waves whose states merge in LDS; the RMS statistic is one wave reduction;
// the interleaved RoPE pairs of the trailing slice stay inside a lane.
#include "common.h"
#include "kernels.h"

namespace csa {
namespace {

constexpr int kMaxWavesPerEntry = 8;

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
    t.live = true;
  } else {
    if (w >= a.B) return t;
    const int p = a.pos[w];
    t.b = w;
    if (p < 0 || (p + 1) % a.ratio != 0) return t;
    t.e = p / a.ratio;
    t.live = t.e < a.out_cap;
  }
  return t;
}

// Row of token `tok` inside a sequence's span (span mode) or ring (ring mode).
__device__ __forceinline__ int64_t token_row(const CompressArgs& a, int64_t tok) {
  return a.pos == nullptr ? tok - a.tok0 : tok % a.T;
}

template <int CPL, bool BF16>
__device__ __forceinline__ void load_lane(const void* base, int64_t off, float (&v)[CPL]) {
  if constexpr (BF16) {
    const uint16_t* p = static_cast<const uint16_t*>(base) + off;
    if constexpr (CPL == 8) {
      uint4 u = *reinterpret_cast<const uint4*>(p);
      uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) { v[2 * i] = bf16_lo(w[i]); v[2 * i + 1] = bf16_hi(w[i]); }
    } else if constexpr (CPL == 4) {
      uint2 u = *reinterpret_cast<const uint2*>(p);
      v[0] = bf16_lo(u.x); v[1] = bf16_hi(u.x); v[2] = bf16_lo(u.y); v[3] = bf16_hi(u.y);
    } else {
      uint32_t u = *reinterpret_cast<const uint32_t*>(p);
      v[0] = bf16_lo(u); v[1] = bf16_hi(u);
    }
  } else {
    const float* p = static_cast<const float*>(base) + off;
#pragma unroll
    for (int i = 0; i < CPL; i += 2) {
      float2 f = *reinterpret_cast<const float2*>(p + i);
      v[i] = f.x; v[i + 1] = f.y;
    }
  }
}

// Fast path: D = 64*CPL, CPL in {2,4,8}.  A block of `wpe` waves builds one
// entry: the candidate rows are split evenly over the waves, every wave runs
// the online softmax over its share with four rows in flight at a time, and
// wave 0 merges the per-wave (max, sum, weighted sum) states through LDS.
template <int CPL, bool BF16>
__global__ __launch_bounds__(kWave* kMaxWavesPerEntry) void compress_lanes(CompressArgs a, int wpe) {
  extern __shared__ float merge[];  // [wpe][3][CPL][64]
  __shared__ float rope_tab[64 * CPL];  // (cos, sin) of every RoPE pair
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const Task task = compress_task(a, blockIdx.x);
  if (!task.live) return;
  const int D = a.D, r = a.ratio, e = task.e;
  const int c0 = lane * CPL;
  const int64_t seq = int64_t(task.b) * a.in_bstride;

  float m[CPL], s[CPL], acc[CPL];
#pragma unroll
  for (int i = 0; i < CPL; ++i) { m[i] = -INFINITY; s[i] = 0.f; acc[i] = 0.f; }

  // candidate c: previous-group token (e-1)*r + c for c < cp, else current token
  const int cp = (a.overlap && e > 0) ? r : 0;
  const int C = cp + r;
  const int per = (C + wpe - 1) / wpe;
  const int cb = wave * per, ce = min(C, cb + per);
  // rows stay in their storage format until absorbed: bf16 pairs or fp32 bits
  constexpr int RW = BF16 ? CPL / 2 : CPL;
  constexpr int kBatch = BF16 ? 8 : 4;
  uint32_t g[kBatch][RW], v[kBatch][RW];
  auto load_raw = [&](const void* base, int64_t off, uint32_t (&w)[RW]) {
    const uint32_t* p = reinterpret_cast<const uint32_t*>(static_cast<const char*>(base) + off * (BF16 ? 2 : 4));
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
      w[0] = *p;
    }
  };
  auto elem = [&](const uint32_t (&w)[RW], int i) -> float {
    if constexpr (BF16) return (i & 1) ? bf16_hi(w[i / 2]) : bf16_lo(w[i / 2]);
    else return __uint_as_float(w[i]);
  };
  // candidates are consecutive tokens from t_first; their rows follow one
  // another in the span, or wrap once around the ring (C <= 2r <= T)
  const int64_t t_first = int64_t(e) * r - cp;
  const int64_t row_first = a.pos == nullptr ? t_first - a.tok0 : t_first % a.T;
  auto load_batch = [&](int c) {
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      if (c + j < ce) {
        const int cc = c + j;
        const bool prev = cc < cp;
        int64_t row = row_first + cc;
        if (a.pos != nullptr && row >= a.T) row -= a.T;
        const int64_t off = seq + row * D + c0;
        load_raw(prev ? a.gate_prev : a.gate, off, g[j]);
        load_raw(prev ? a.kv_prev : a.kv, off, v[j]);
      }
    }
  };
  if (cb < ce) load_batch(cb);

  // RoPE table (one rolled loop, one call site) and gamma while the first
  // rows are in flight
  const int rope0 = D - a.rope_dim;
  for (int i = threadIdx.x; i < a.rope_dim / 2; i += blockDim.x)
    rope_cos_sin(int64_t(e) * r, i, a.rope_dim, a.rope_base, &rope_tab[2 * i], &rope_tab[2 * i + 1]);
  float gam[CPL];
#pragma unroll
  for (int i = 0; i < CPL; ++i) gam[i] = a.gamma[c0 + i];

  for (int c = cb; c < ce; c += kBatch) {
    if (c != cb) load_batch(c);
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      if (c + j >= ce) break;
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const float gl = elem(g[j], i) * kLog2e;
        const float mn = fmaxf(m[i], gl);
        const float keep = fast_exp2(m[i] - mn);  // 0 on the first candidate
        const float pj = fast_exp2(gl - mn);
        s[i] = s[i] * keep + pj;
        acc[i] = acc[i] * keep + pj * elem(v[j], i);
        m[i] = mn;
      }
    }
  }
  if (wpe > 1) {
    float* mine = merge + wave * 3 * CPL * kWave;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      mine[(0 * CPL + i) * kWave + lane] = m[i];
      mine[(1 * CPL + i) * kWave + lane] = s[i];
      mine[(2 * CPL + i) * kWave + lane] = acc[i];
    }
    __syncthreads();
    if (wave != 0) return;
    for (int w = 1; w < wpe; ++w) {
      const float* o = merge + w * 3 * CPL * kWave;
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const float mw = o[(0 * CPL + i) * kWave + lane];
        if (mw == -INFINITY) continue;  // that wave had no candidate
        const float mn = fmaxf(m[i], mw);
        const float f0 = fast_exp2(m[i] - mn), f1 = fast_exp2(mw - mn);
        s[i] = s[i] * f0 + o[(1 * CPL + i) * kWave + lane] * f1;
        acc[i] = acc[i] * f0 + o[(2 * CPL + i) * kWave + lane] * f1;
        m[i] = mn;
      }
    }
  }

  if (wpe == 1) __syncthreads();  // publishes the RoPE table (merge's barrier does it otherwise)
  float y[CPL];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < CPL; ++i) { y[i] = acc[i] / s[i]; ss += y[i] * y[i]; }
  ss = wave_sum(ss);
  const float inv_rms = rsqrtf(ss / float(D) + a.eps);
#pragma unroll
  for (int i = 0; i < CPL; ++i) y[i] *= inv_rms * gam[i];
  if (c0 + CPL > rope0) {
#pragma unroll
    for (int i = 0; i < CPL / 2; ++i) {
      const int ch = c0 + 2 * i;
      if (ch < rope0) continue;
      const float cs = rope_tab[ch - rope0], sn = rope_tab[ch - rope0 + 1];
      const float x0 = y[2 * i], x1 = y[2 * i + 1];
      y[2 * i] = x0 * cs - x1 * sn;
      y[2 * i + 1] = x0 * sn + x1 * cs;
    }
  }

  const int64_t o = int64_t(task.b) * a.out_bstride + int64_t(e) * D + c0;
  if (a.out_dtype == CSA_BF16) {
    uint16_t* dst = static_cast<uint16_t*>(a.out) + o;
    if constexpr (CPL == 8) {
      uint4 u{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]), pack_bf16x2(y[4], y[5]), pack_bf16x2(y[6], y[7])};
      *reinterpret_cast<uint4*>(dst) = u;
    } else if constexpr (CPL == 4) {
      *reinterpret_cast<uint2*>(dst) = uint2{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
    } else {
      *reinterpret_cast<uint32_t*>(dst) = pack_bf16x2(y[0], y[1]);
    }
  } else {
    float* dst = static_cast<float*>(a.out) + o;
#pragma unroll
    for (int i = 0; i < CPL; i += 2) *reinterpret_cast<float2*>(dst + i) = float2{y[i], y[i + 1]};
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
    rope_cos_sin(int64_t(e) * r, i, a.rope_dim, a.rope_base, &cs, &sn);
    const float x0 = ybuf[rope0 + 2 * i], x1 = ybuf[rope0 + 2 * i + 1];
    ybuf[rope0 + 2 * i] = x0 * cs - x1 * sn;
    ybuf[rope0 + 2 * i + 1] = x0 * sn + x1 * cs;
  }
  __syncthreads();
  const int64_t o = int64_t(task.b) * a.out_bstride + int64_t(e) * D;
  for (int c = lane; c < D; c += kWave) store_elem(a.out, a.out_dtype, o + c, ybuf[c]);
}

}  // namespace

hipError_t launch_compress(const CompressArgs& a, hipStream_t stream) {
  const int tasks = a.pos == nullptr ? a.B * a.n_entries : a.B;
  if (tasks == 0) return hipSuccess;
  const int cpl = a.D / kWave;
  auto al = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
  const int in_es = a.in_dtype == CSA_BF16 ? 2 : 4, out_es = a.out_dtype == CSA_BF16 ? 2 : 4;
  const bool lanes_ok = (a.D % kWave == 0) && (cpl == 2 || cpl == 4 || cpl == 8) && al(a.kv) && al(a.gate) &&
                        al(a.kv_prev) && al(a.gate_prev) && al(a.out) && (a.in_bstride * in_es) % 16 == 0 &&
                        (a.out_bstride * out_es) % 16 == 0;
  if (lanes_ok) {
    // one wave per 8 candidate rows (one load batch), at most 8 waves
    const int cand = (1 + a.overlap) * a.ratio;
    int wpe = (cand + 7) / 8;
    wpe = wpe < 1 ? 1 : (wpe > kMaxWavesPerEntry ? kMaxWavesPerEntry : wpe);
    const dim3 grid(tasks), block(kWave * wpe);
    const size_t lds = wpe > 1 ? size_t(wpe) * 3 * cpl * kWave * sizeof(float) : 0;
    const bool bf = a.in_dtype == CSA_BF16;
#define CSA_COMPRESS_CASE(C)                                                                  \
  if (cpl == C) {                                                                             \
    if (bf) hipLaunchKernelGGL((compress_lanes<C, true>), grid, block, lds, stream, a, wpe);  \
    else hipLaunchKernelGGL((compress_lanes<C, false>), grid, block, lds, stream, a, wpe);    \
  }
    CSA_COMPRESS_CASE(2)
    CSA_COMPRESS_CASE(4)
    CSA_COMPRESS_CASE(8)
#undef CSA_COMPRESS_CASE
  } else {
    hipLaunchKernelGGL(compress_any, dim3(tasks), dim3(kWave), a.D * sizeof(float), stream, a);
  }
  return hipGetLastError();
}

}  // namespace csa
