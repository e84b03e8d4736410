// Joint-softmax attention over window rows plus compressed rows, with a
// per-head sink and an inverse RoPE on the output (CSA and HCA).
//
// "DeepSeek-V4-Flash 架构：一个 token 的旅程", sections "局部和压缩记忆，共用一次
// 归一化" (one candidate set, one normalisation, the sink adds to the
// denominator only), "输出投影也分组，并且降低中间维度" (inverse RoPE of the
// output) and "长上下文时，先数真正访问的条目" (QK and weighted-V are the two
// multiply-add stages); "LLM Atlas: DeepSeek" §19 (HCA attends to every
// compressed entry, CSA to the top-k); "Lab tổng hợp DeepSeek-V4.1-Flash",
// section "3 Giải pháp" (all query heads share one K/V head).
//
// Matrix-core path (bf16, 64 heads, D = 512).  All 64 heads of a query share
// every K=V row, so one workgroup (4 waves x 16 heads) gathers each 32-row
// candidate tile once into LDS -- row-major for the QK product and transposed
// for the PV product -- and runs both products on 16x16x32 bf16 MFMA:
//   S^T[rows x heads] = K . Q^T   (A = K rows from LDS, B = Q held in VGPRs)
//   O^T[dims x heads] += V^T . P^T (A = V^T from LDS, B = P straight from the
//                                  S^T accumulators, no shuffle)
// The tile's A rows are permuted so that each lane's eight S^T results are
// eight consecutive candidate rows, exactly the K-slice its P^T operand
// needs.  Softmax state (running max, partial sums) is per head = per lane,
// so the rescale of the 128 output accumulators is lane-local.
//
// Few queries (decode) split the candidate list over workgroups; each writes
// an unnormalised partial (O, max, sum) and a combine kernel merges the
// splits with the sink and applies the inverse RoPE.  With one split the sink
// seeds the running max/sum and the kernel finishes the output itself.
#include "common.h"
#include "kernels.h"

namespace csa {
namespace {

constexpr int kH = 64;      // heads on the matrix-core path
constexpr int kD = 512;     // K=V row width on the matrix-core path
constexpr int kTile = 32;   // candidate rows per tile
constexpr int kKPitch = kD + 8;     // bf16 elements per K row in LDS (16 B pad)
// K tile in LDS: 16-byte chunk c of row r sits at chunk c ^ (4 * ((r >> 4) & 1)).
// With the 16-byte row pad, the 16 rows one S^T fragment reads then start on
// 16 different bank groups, so its 64 lanes spread evenly over the banks.
__device__ __forceinline__ int kt_off(int row, int chunk) {
  return row * kKPitch + ((chunk ^ (((row >> 4) & 1) << 2)) << 3);
}
// V^T in LDS: row d (one dim, 32 candidate rows) starts at d*32 + (d/8)*8
// elements; the 16-byte skew per 8 dims spreads the transposed tile writes
// (lanes 8 dims apart) over all LDS banks.
__device__ __forceinline__ int vt_off(int d) { return d * kTile + (d >> 3) * 8; }
constexpr int kVtElems = kD * kTile + (kD / 8) * 8;
constexpr int kMinSplitRows = 64;
constexpr int kTargetBlocks = 256;
constexpr int kMaxChunk = 4352;   // CSA candidates of one block, resolved in LDS
constexpr int kMaxSplits = 256;

struct Cand {
  int n_win;
  int64_t n_sel;
  int64_t p;
  int s0;  // ring slot of the oldest window row
};

__device__ __forceinline__ Cand candidates(const AttnArgs& a, bool hca, int64_t qi) {
  Cand c;
  const int p = a.pos[qi];
  c.p = p;
  c.s0 = 0;
  if (p < 0) { c.n_win = 0; c.n_sel = 0; return c; }
  c.n_win = p + 1 < a.window ? p + 1 : a.window;
  c.s0 = int((int64_t(p) - c.n_win + 1) % a.Wcap);
  if (hca) {
    const int64_t nv = (int64_t(p) + 1) / a.ratio;
    c.n_sel = nv < a.Ncap ? nv : a.Ncap;
  } else {
    c.n_sel = a.k;
  }
  return c;
}

// Element offset of candidate j's row, or -1 when it does not exist.
__device__ __forceinline__ int64_t cand_row(const AttnArgs& a, bool hca, const Cand& c, int64_t qi, int b,
                                            int64_t j, bool* from_win) {
  if (j < c.n_win) {
    *from_win = true;
    const int64_t pp = c.p - c.n_win + 1 + j;
    return (int64_t(b) * a.Wcap + pp % a.Wcap) * a.D;
  }
  *from_win = false;
  const int64_t i = j - c.n_win;
  if (i >= c.n_sel) return -1;
  const int64_t e = hca ? i : int64_t(a.idx[qi * a.k + i]);
  if (e < 0 || e >= a.Ncap) return -1;
  return (int64_t(b) * a.Ncap + e) * a.D;
}

// Candidate code: >= 0 compressed entry, <= -2 window ring slot (-2 - slot),
// -1 no row.
__device__ __forceinline__ int cand_code(const AttnArgs& a, bool hca, const Cand& c, int64_t qi, int64_t j) {
  if (j < c.n_win) {
    const int slot = c.s0 + int(j);  // j < window <= Wcap: at most one wrap
    return -2 - (slot >= a.Wcap ? slot - a.Wcap : slot);
  }
  const int64_t i = j - c.n_win;
  if (i >= c.n_sel) return -1;
  const int64_t e = hca ? i : int64_t(a.idx[qi * a.k + i]);
  return (e >= 0 && e < a.Ncap) ? int(e) : -1;
}

// ---------------------------------------------------------------------------
// Matrix-core kernel: grid (B*S, nsplit), 256 threads.
// ---------------------------------------------------------------------------
template <bool HCA, bool SPLIT>
__global__ __launch_bounds__(256) void attn_mfma(AttnArgs a, int nsplit, int chunk_rows) {
  __shared__ __attribute__((aligned(16))) uint16_t Kt[kTile * kKPitch];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[kVtElems];
  __shared__ float rope_cs[kD];
  __shared__ unsigned char valid[kTile];
  __shared__ int codes[HCA ? 1 : kMaxChunk];

  const int64_t qi = blockIdx.x;
  const int split = blockIdx.y;
  const int b = int(qi / a.S);
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int g = lane / 16, r16 = lane % 16;
  const int head = wave * 16 + r16;
  const Cand c = candidates(a, HCA, qi);
  const int64_t n_cand = c.n_win + c.n_sel;
  const int64_t j_begin = int64_t(split) * chunk_rows;
  const int n_rows = int(j_begin < n_cand ? (n_cand - j_begin < chunk_rows ? n_cand - j_begin : chunk_rows) : 0);
  const uint16_t* win = static_cast<const uint16_t*>(a.win) + int64_t(b) * a.Wcap * kD;
  const uint16_t* cmp = static_cast<const uint16_t*>(a.cmp) + int64_t(b) * a.Ncap * kD;

  // Q^T operand: Q[head][ks*32 + g*8 .. +7], 16 K-steps.
  bf16x8 qb[16];
  {
    const uint16_t* q = static_cast<const uint16_t*>(a.q) + (qi * kH + head) * kD + g * 8;
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) qb[ks] = as_bf16x8(*reinterpret_cast<const uint4*>(q + ks * 32));
  }
  // CSA: resolve the chunk's selections once, so that tile gathers never wait
  // on a dependent index load.
  if constexpr (!HCA) {
    for (int j = tid; j < n_rows; j += 256) codes[j] = cand_code(a, false, c, qi, j_begin + j);
    __syncthreads();
  }

  const float qk_scale = a.scale * kLog2e;
  const float sink2 = a.sink[head] * kLog2e;
  // m_run is a reference maximum: it moves only when some head's running max
  // exceeds it by more than 2^8 (lazy rescale), so exponentials stay <= 256
  // and the 128-accumulator rescale runs on very few tiles.
  float m_run, l_run;
  if constexpr (!SPLIT) { m_run = sink2; l_run = g == 0 ? 1.f : 0.f; }
  else { m_run = -1e30f; l_run = 0.f; }
  floatx4 acc[32];
#pragma unroll
  for (int mt = 0; mt < 32; ++mt) acc[mt] = floatx4{0.f, 0.f, 0.f, 0.f};

  // gather geometry: thread owns 8 dims (dc*8..) of 8 rows (rg*8..) of a tile
  const int dc = tid % 64, rg = tid / 64;
  auto gather = [&](int jl0, uint4 (&v)[8]) -> unsigned {
    unsigned mask = 0;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int jl = jl0 + rg * 8 + r;
      int code = -1;
      if (jl < n_rows) code = HCA ? cand_code(a, true, c, qi, j_begin + jl) : codes[jl];
      const uint16_t* src = code >= 0 ? cmp + int64_t(code) * kD : (code <= -2 ? win + int64_t(-2 - code) * kD : nullptr);
      if (src != nullptr) {
        v[r] = *reinterpret_cast<const uint4*>(src + dc * 8);
        mask |= 1u << r;
      } else {
        v[r] = uint4{0, 0, 0, 0};
      }
    }
    return mask;
  };

  uint4 v[8];
  unsigned vmask = n_rows > 0 ? gather(0, v) : 0u;
  for (int jl0 = 0; jl0 < n_rows; jl0 += kTile) {
#pragma unroll
    for (int r = 0; r < 8; ++r)
      *reinterpret_cast<uint4*>(&Kt[kt_off(rg * 8 + r, dc)]) = v[r];
    // transpose the 8x8 block: Vt[dim][rows rg*8 .. +7]
#pragma unroll
    for (int dd = 0; dd < 8; ++dd) {
      uint32_t w4[4];
#pragma unroll
      for (int rp = 0; rp < 4; ++rp) {
        const uint32_t* a0 = reinterpret_cast<const uint32_t*>(&v[2 * rp]);
        const uint32_t* a1 = reinterpret_cast<const uint32_t*>(&v[2 * rp + 1]);
        const uint32_t x0 = a0[dd / 2], x1 = a1[dd / 2];
        w4[rp] = (dd & 1) ? ((x0 >> 16) | (x1 & 0xffff0000u)) : ((x0 & 0xffffu) | (x1 << 16));
      }
      *reinterpret_cast<uint4*>(&Vt[vt_off(dc * 8 + dd) + rg * 8]) = uint4{w4[0], w4[1], w4[2], w4[3]};
    }
    if (dc == 0) {
#pragma unroll
      for (int r = 0; r < 8; ++r) valid[rg * 8 + r] = (vmask >> r) & 1u;
    }
    __syncthreads();
    // the next tile's rows stream in while this one is multiplied
    if (jl0 + kTile < n_rows) vmask = gather(jl0 + kTile, v);

    // S^T tiles: tile t covers candidate rows (m/4)*8 + t*4 + m%4
    float s8[8];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int arow = (r16 / 4) * 8 + t * 4 + (r16 % 4);
      floatx4 st = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 16; ++ks)
        st = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            as_bf16x8(*reinterpret_cast<const uint4*>(&Kt[kt_off(arow, ks * 4 + g)])), qb[ks], st, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) s8[t * 4 + i] = st[i];
    }
    // lane holds rows g*8 + 0..7 of head `head`
    float tmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      s8[i] = valid[g * 8 + i] ? s8[i] * qk_scale : -INFINITY;
      tmax = fmaxf(tmax, s8[i]);
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, kWave));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave));
    if (__any(tmax > m_run + 8.f)) {  // wave-uniform: rescale every head of the wave
      const float m_new = fmaxf(m_run, tmax);
      const float alpha = fast_exp2(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int mt = 0; mt < 32; ++mt) acc[mt] *= alpha;
      m_run = m_new;
    }
    float psum = 0.f;
    uint32_t pw[4];
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
      const float p0 = fast_exp2(s8[i] - m_run), p1 = fast_exp2(s8[i + 1] - m_run);
      psum += p0 + p1;
      pw[i / 2] = pack_bf16x2(p0, p1);
    }
    l_run += psum;
    const bf16x8 pb = as_bf16x8(uint4{pw[0], pw[1], pw[2], pw[3]});
#pragma unroll
    for (int mt = 0; mt < 32; ++mt) {
      const bf16x8 va = as_bf16x8(*reinterpret_cast<const uint4*>(&Vt[vt_off(mt * 16 + r16) + g * 8]));
      acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb, acc[mt], 0, 0, 0);
    }
    __syncthreads();
  }

  l_run += __shfl_xor(l_run, 16, kWave);
  l_run += __shfl_xor(l_run, 32, kWave);
  // lane holds O^T[dims mt*16 + g*4 + i][head]
  if constexpr (!SPLIT) {
    const int rope0 = kD - a.rope_dim;
    for (int i = tid; i < a.rope_dim / 2; i += 256) {
      float cs, sn;
      rope_cos_sin(c.p, i, a.rope_dim, a.rope_base, &cs, &sn);
      rope_cs[2 * i] = cs;
      rope_cs[2 * i + 1] = sn;
    }
    __syncthreads();
    const float inv_l = 1.f / l_run;
    const int64_t obase = (qi * kH + head) * kD;
#pragma unroll
    for (int mt = 0; mt < 32; ++mt) {
      float o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = acc[mt][i] * inv_l;
      const int d0 = mt * 16 + g * 4;
      if (d0 >= rope0 && c.p >= 0) {
#pragma unroll
        for (int i = 0; i < 4; i += 2) {
          const int pi = (d0 + i - rope0) / 2;
          const float cs = rope_cs[2 * pi], sn = rope_cs[2 * pi + 1];
          const float x0 = o[i], x1 = o[i + 1];
          o[i] = x0 * cs + x1 * sn;
          o[i + 1] = x1 * cs - x0 * sn;
        }
      }
      if (a.out_dtype == CSA_BF16) {
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + obase + d0) =
            uint2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
      } else {
        *reinterpret_cast<float4*>(static_cast<float*>(a.out) + obase + d0) = float4{o[0], o[1], o[2], o[3]};
      }
    }
  } else {
    float* ws_o = static_cast<float*>(a.ws);
    float* ws_ml = ws_o + int64_t(a.B) * a.S * nsplit * kH * kD;
    const int64_t slot = (qi * nsplit + split) * kH + head;
#pragma unroll
    for (int mt = 0; mt < 32; ++mt)
      *reinterpret_cast<floatx4*>(ws_o + slot * kD + mt * 16 + g * 4) = acc[mt];
    if (g == 0) {
      ws_ml[2 * slot] = m_run;
      ws_ml[2 * slot + 1] = l_run;
    }
  }
}

// Merge the splits of one (query, head) with the sink; inverse RoPE; store.
// grid (B*S, H/4), 256 threads: one wave per head, lane owns 8 dims; the
// split factors are formed once per head and every split's partial is
// fetched with several loads in flight.
__global__ __launch_bounds__(256) void attn_combine(AttnArgs a, int nsplit) {
  __shared__ float rope_cs[kD];
  __shared__ float fac[4][kMaxSplits];
  const int64_t qi = blockIdx.x;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int h = blockIdx.y * 4 + wave;
  const int p = a.pos[qi];
  for (int i = tid; i < a.rope_dim / 2; i += 256) {
    float cs, sn;
    rope_cos_sin(p, i, a.rope_dim, a.rope_base, &cs, &sn);
    rope_cs[2 * i] = cs;
    rope_cs[2 * i + 1] = sn;
  }
  const float* ws_o = static_cast<const float*>(a.ws);
  const float* ws_ml = ws_o + int64_t(a.B) * a.S * nsplit * kH * kD;
  const float sink2 = a.sink[h] * kLog2e;
  float mx = sink2;
  for (int s = lane; s < nsplit; s += kWave) mx = fmaxf(mx, ws_ml[2 * ((qi * nsplit + s) * kH + h)]);
  mx = wave_max(mx);
  float lsum = 0.f;
  for (int s = lane; s < nsplit; s += kWave) {
    const int64_t slot = (qi * nsplit + s) * kH + h;
    const float f = fast_exp2(ws_ml[2 * slot] - mx);
    fac[wave][s] = f;
    lsum += ws_ml[2 * slot + 1] * f;
  }
  const float L = wave_sum(lsum) + fast_exp2(sink2 - mx);
  __syncthreads();

  const int d0 = lane * 8;
  float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  constexpr int kBatch = 8;
  for (int s0 = 0; s0 < nsplit; s0 += kBatch) {
    float4 u[kBatch][2];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      if (s0 + j < nsplit) {
        const float4* src = reinterpret_cast<const float4*>(ws_o + ((qi * nsplit + s0 + j) * kH + h) * kD + d0);
        u[j][0] = src[0];
        u[j][1] = src[1];
      }
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      if (s0 + j >= nsplit) break;
      const float f = fac[wave][s0 + j];
      o[0] += f * u[j][0].x; o[1] += f * u[j][0].y; o[2] += f * u[j][0].z; o[3] += f * u[j][0].w;
      o[4] += f * u[j][1].x; o[5] += f * u[j][1].y; o[6] += f * u[j][1].z; o[7] += f * u[j][1].w;
    }
  }
  const float inv = 1.f / L;
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] *= inv;
  const int rope0 = kD - a.rope_dim;
  if (d0 >= rope0 && p >= 0) {
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
      const int pi = (d0 + i - rope0) / 2;
      const float cs = rope_cs[2 * pi], sn = rope_cs[2 * pi + 1];
      const float x0 = o[i], x1 = o[i + 1];
      o[i] = x0 * cs + x1 * sn;
      o[i + 1] = x1 * cs - x0 * sn;
    }
  }
  const int64_t obase = (qi * kH + h) * kD + d0;
  if (a.out_dtype == CSA_BF16) {
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.out) + obase) =
        uint4{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]), pack_bf16x2(o[4], o[5]), pack_bf16x2(o[6], o[7])};
  } else {
    float4* dst = reinterpret_cast<float4*>(static_cast<float*>(a.out) + obase);
    dst[0] = float4{o[0], o[1], o[2], o[3]};
    dst[1] = float4{o[4], o[5], o[6], o[7]};
  }
}

// ---------------------------------------------------------------------------
// Vector-ALU kernel for other shapes: one wave per (query, head), online
// softmax over the candidates, D <= 1024.
// ---------------------------------------------------------------------------
template <bool HCA>
__global__ __launch_bounds__(kWave) void attn_any(AttnArgs a) {
  extern __shared__ float obuf[];  // D floats
  const int64_t qi = blockIdx.x;
  const int h = blockIdx.y, lane = threadIdx.x;
  const int b = int(qi / a.S);
  const int D = a.D;
  const Cand c = candidates(a, HCA, qi);
  const int64_t n_cand = c.n_win + c.n_sel;
  constexpr int kMaxPer = 1024 / kWave;
  float q[kMaxPer], o[kMaxPer];
  const int64_t qoff = (qi * a.H + h) * D;
#pragma unroll
  for (int i = 0; i < kMaxPer; ++i) {
    const int d = lane + i * kWave;
    q[i] = d < D ? load_elem(a.q, a.dtype, qoff + d) : 0.f;
    o[i] = 0.f;
  }
  const float qk_scale = a.scale * kLog2e;
  float m = a.sink[h] * kLog2e, l = 1.f;
  for (int64_t j = 0; j < n_cand; ++j) {
    bool fw;
    const int64_t off = cand_row(a, HCA, c, qi, b, j, &fw);
    if (off < 0) continue;
    const void* src = fw ? a.win : a.cmp;
    float rowv[kMaxPer];
    float dot = 0.f;
#pragma unroll
    for (int i = 0; i < kMaxPer; ++i) {
      const int d = lane + i * kWave;
      rowv[i] = d < D ? load_elem(src, a.dtype, off + d) : 0.f;
      dot += q[i] * rowv[i];
    }
    const float s = wave_sum(dot) * qk_scale;
    const float mn = fmaxf(m, s);
    const float alpha = fast_exp2(m - mn), pj = fast_exp2(s - mn);
    l = l * alpha + pj;
#pragma unroll
    for (int i = 0; i < kMaxPer; ++i) o[i] = o[i] * alpha + pj * rowv[i];
    m = mn;
  }
#pragma unroll
  for (int i = 0; i < kMaxPer; ++i) {
    const int d = lane + i * kWave;
    if (d < D) obuf[d] = o[i] / l;
  }
  __syncthreads();
  const int rope0 = D - a.rope_dim;
  if (c.p >= 0) {
    for (int i = lane; i < a.rope_dim / 2; i += kWave) {
      float cs, sn;
      rope_cos_sin(c.p, i, a.rope_dim, a.rope_base, &cs, &sn);
      const float x0 = obuf[rope0 + 2 * i], x1 = obuf[rope0 + 2 * i + 1];
      obuf[rope0 + 2 * i] = x0 * cs + x1 * sn;
      obuf[rope0 + 2 * i + 1] = x1 * cs - x0 * sn;
    }
  }
  __syncthreads();
  for (int d = lane; d < D; d += kWave) store_elem(a.out, a.out_dtype, qoff + d, obuf[d]);
}

}  // namespace

AttnPlan plan_attn(int B, int S, int H, int D, int max_cand, int dtype, bool hca) {
  AttnPlan p{false, 1, 0, 0};
  p.mfma = dtype == CSA_BF16 && H == kH && D == kD;
  if (!p.mfma) return p;
  const int64_t nq = int64_t(B) * S;
  int64_t want = nq > 0 ? (kTargetBlocks + nq - 1) / nq : 1;
  const int64_t most = (max_cand + kMinSplitRows - 1) / kMinSplitRows;
  if (want > most) want = most;
  if (want > kMaxSplits) want = kMaxSplits;
  if (want < 1) want = 1;
  int64_t rows = (max_cand + want - 1) / want;
  rows = (rows + kTile - 1) / kTile * kTile;
  if (rows < kTile) rows = kTile;
  if (!hca && rows > kMaxChunk) rows = kMaxChunk;
  p.chunk_rows = int(rows);
  p.nsplit = int((max_cand + rows - 1) / rows);
  if (p.nsplit < 1) p.nsplit = 1;
  if (p.nsplit > 1)
    p.ws_bytes = size_t(nq) * p.nsplit * kH * (size_t(kD) + 2) * sizeof(float);
  return p;
}

hipError_t launch_attn(const AttnArgs& a, const AttnPlan& plan, bool hca, hipStream_t stream) {
  const int64_t nq = int64_t(a.B) * a.S;
  if (nq == 0) return hipSuccess;
  if (plan.mfma) {
    const dim3 grid(unsigned(nq), plan.nsplit);
    const bool split = plan.nsplit > 1;
    if (hca && split) hipLaunchKernelGGL((attn_mfma<true, true>), grid, dim3(256), 0, stream, a, plan.nsplit, plan.chunk_rows);
    else if (hca) hipLaunchKernelGGL((attn_mfma<true, false>), grid, dim3(256), 0, stream, a, plan.nsplit, plan.chunk_rows);
    else if (split) hipLaunchKernelGGL((attn_mfma<false, true>), grid, dim3(256), 0, stream, a, plan.nsplit, plan.chunk_rows);
    else hipLaunchKernelGGL((attn_mfma<false, false>), grid, dim3(256), 0, stream, a, plan.nsplit, plan.chunk_rows);
    if (plan.nsplit > 1)
      hipLaunchKernelGGL(attn_combine, dim3(unsigned(nq), kH / 4), dim3(256), 0, stream, a, plan.nsplit);
  } else {
    const dim3 grid(unsigned(nq), a.H);
    if (hca) hipLaunchKernelGGL((attn_any<true>), grid, dim3(kWave), a.D * sizeof(float), stream, a);
    else hipLaunchKernelGGL((attn_any<false>), grid, dim3(kWave), a.D * sizeof(float), stream, a);
  }
  return hipGetLastError();
}

}  // namespace csa
