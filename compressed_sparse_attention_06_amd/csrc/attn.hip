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
// every K=V row.  A workgroup of eight waves (two per SIMD) takes one query,
// or one split of its candidate list, in tiles of 32 candidate rows, with the
// waves specialised:
//   * QK waves 0..3: wave w holds Q^T of heads 32*(w&1)..+32 in VGPRs and
//     scores rows 16*(w>>1)..+16 of each tile on 16x16x32 bf16 MFMA
//     (S^T = K . Q^T), then writes P = exp2(S - m) to LDS as bf16;
//   * PV waves 4..7: wave 4+v owns O^T for dims 128v..+128 and all 64 heads
//     and accumulates O^T += V^T . P^T one tile behind the QK waves; its V^T
//     operand comes from the row-major tile through the transposing LDS read
//     (ds_read_b64_tr_b16).
// On each SIMD one QK and one PV wave share the matrix core, so the softmax
// arithmetic of one overlaps the products of the other.  Tile rows are copied
// HBM -> LDS by the load unit itself (one 1 KiB row per wave instruction),
// two tiles ahead, into a ring of four tile buffers; one barrier per tile
// step orders everything.
//
// Softmax reference: every head accumulates exp2(s - m) against a fixed
// reference m = its sink logit (log2 units), so no maxima are exchanged and
// O is never rescaled; fp32 accumulators and bf16 P hold values up to 2^64
// times the reference with room to spare.  Should a score exceed the
// reference by more than that headroom, the whole pass is repeated with the
// true maximum as the reference (never for ordinary data).
//
// Few queries (decode) split the candidate list over workgroups; each writes
// an unnormalised partial (O, m, sum) and a combine kernel merges the splits
// with the sink and applies the inverse RoPE.  With one split the sink's
// unit term is part of the sum and the kernel finishes the output itself.
#include "common.h"
#include "kernels.h"
#include "kv4.h"

namespace csa {
namespace {

constexpr int kH = 64;      // heads on the matrix-core path
constexpr int kD = 512;     // K=V row width on the matrix-core path
constexpr int kT = 32;      // candidate rows per tile
constexpr int kBufs = 4;    // tile ring: PV tile, QK tile, two copies in flight
constexpr int kWaves = 8;   // 4 QK + 4 PV waves
constexpr int kThreads = kWaves * kWave;
constexpr int kCopyRows = kT / kWaves;  // rows each wave copies per tile
constexpr int kRowBytes = kD * 2;
// LDS tile layout (measured bank-conflict free on gfx950 for both the
// 128-bit K reads and the transposing V reads): row pitch 1 KiB + 32 B, and
// in rows whose bits 2 and 3 differ, 16-byte chunk c of the row is stored at
// chunk c ^ 8.  Every per-step offset is then an immediate added to one of
// two per-lane bases.
constexpr int kPitch = kRowBytes + 32;
__device__ __forceinline__ int row_flip(int r) { return ((r >> 2) ^ (r >> 3)) & 1; }
constexpr int kPPitch = kT + 8;   // bf16 per head row of P in LDS (80 B: 8 heads on distinct banks)
constexpr int kAheadK = 4;        // K operand prefetch distance, in K-steps
constexpr int kAheadV = 3;        // V^T operand prefetch distance, in dim tiles
constexpr float kHeadroom = 64.f;  // log2 of the largest P relative to the reference
constexpr int kMinSplitRows = 64;
constexpr int kSplitGrain = 32;
constexpr int kTargetBlocks = 256;
constexpr int kMaxChunk = 1024;   // CSA candidates of one block, resolved in LDS
constexpr int kMaxSplits = 256;

// One 1 KiB row copy HBM -> LDS through the load unit: lane l moves the 16
// bytes at row + voff to LDS address lds_row + 16 l (M0 carries lds_row).
// Written as asm so that the compiler does not order LDS reads of other tile
// buffers behind it; the kernel waits for these copies itself before the
// barrier that publishes a tile.  The compiler's hazard checks do not see
// into asm, so the asm supplies the wait states itself: a vector-memory
// instruction must not read an SGPR that a VALU instruction (readlane,
// readfirstlane) wrote fewer than 5 instructions before, and an M0 write
// needs one wait state before an LDS-DMA load.
__device__ __forceinline__ void copy_row_to_lds(const void* row, uint32_t voff, uint32_t lds_row) {
  // the row address is wave-uniform; readfirstlane states it so it can sit in SGPRs
  const uint64_t r = reinterpret_cast<uint64_t>(row);
  const uint64_t su = uint64_t(uint32_t(__builtin_amdgcn_readfirstlane(uint32_t(r)))) |
                      (uint64_t(uint32_t(__builtin_amdgcn_readfirstlane(uint32_t(r >> 32)))) << 32);
  asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(su), "{m0}"(lds_row) : "memory");
}
// s_waitcnt with only the vector-memory count set (expcnt, lgkmcnt: no wait)
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) shortx4 lds_shortx4;
typedef __attribute__((address_space(3))) void lds_void;

// 4 x 16-bit transposing LDS read: within each 16-lane group, lane j gets
// element j%4 of the 8-byte chunks addressed by lanes 4i + j/4 (i = 0..3).
__device__ __forceinline__ uint2 lds_read_tr16(const unsigned char* p) {
  const shortx4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(p));
  uint2 r;
  __builtin_memcpy(&r, &v, 8);
  return r;
}

// Finite reference of a head: its sink logit in log2 units (0 if the sink is
// not finite; a -inf sink then contributes exp2(-inf) = 0 to the sum).
__device__ __forceinline__ float sink_ref(const float* sink, int h) {
  const float s2 = sink[h] * kLog2e;
  return (s2 > -1e30f && s2 < 1e30f) ? s2 : 0.f;
}

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
  if (a.pt.pages) {
    const int64_t r = paged_row(a.pt, b, e);
    return r < 0 ? -1 : r * a.D;
  }
  return (int64_t(b) * a.Ncap + e) * a.D;
}

// Candidate code: >= 0 compressed row (the entry, or its pool row in a paged
// cache), <= -2 window ring slot (-2 - slot), -1 no row.
__device__ __forceinline__ int cand_code(const AttnArgs& a, bool hca, const Cand& c, int64_t qi, int64_t j) {
  if (j < c.n_win) {
    const int slot = c.s0 + int(j);  // j < window <= Wcap: at most one wrap
    return -2 - (slot >= a.Wcap ? slot - a.Wcap : slot);
  }
  const int64_t i = j - c.n_win;
  if (i >= c.n_sel) return -1;
  const int64_t e = hca ? i : int64_t(a.idx[qi * a.k + i]);
  if (e < 0 || e >= a.Ncap) return -1;
  if (a.pt.pages) return int(paged_row(a.pt, int(qi / a.S), e));  // -1 when unallocated
  return int(e);
}

// Split partials.  Split (qi, split) stores, per head h, its part of the
// softmax numerator O_h (512 dims) and denominator l_h against the reference
// m_h, as O_h / l_h in fp16 scaled by 2^-e_h (e_h >= 0 the smallest exponent
// that keeps the head's largest value below 2^15): 64 blocks of 1 KiB, block
// (v, dp, ht) holding at lane l's 16 bytes dims 128v + 32dp + 4(l/16) + 0..3
// and the same dims + 16 of head 16ht + l%16 -- the PV waves' accumulator
// fragments, so that both the stores and the combine's loads are whole
// contiguous blocks.  After all partials: (m_h, l_h, e_h, 0) per (qi, split,
// head) in fp32.  Normalising before rounding bounds every stored value by
// the largest |V| entry, so fp16's 11-bit significand sets the error.
constexpr int kPartialVecs = kH * kD * 2 / 16;  // 16-byte units per split partial
__device__ __forceinline__ int partial_block(int v, int dp, int ht) { return (v * 4 + dp) * 4 + ht; }
__device__ __forceinline__ float* partial_ml(const AttnArgs& a, int nsplit) {
  return reinterpret_cast<float*>(static_cast<char*>(a.ws) + size_t(a.B) * a.S * nsplit * kPartialVecs * 16);
}
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  const _Float16 a = static_cast<_Float16>(lo), b = static_cast<_Float16>(hi);  // round to nearest even
  uint16_t ua, ub;
  __builtin_memcpy(&ua, &a, 2);
  __builtin_memcpy(&ub, &b, 2);
  return uint32_t(ua) | (uint32_t(ub) << 16);
}
__device__ __forceinline__ float f16_lo(uint32_t pair) {
  const uint16_t u = uint16_t(pair);
  _Float16 h;
  __builtin_memcpy(&h, &u, 2);
  return static_cast<float>(h);
}
__device__ __forceinline__ float f16_hi(uint32_t pair) {
  const uint16_t u = uint16_t(pair >> 16);
  _Float16 h;
  __builtin_memcpy(&h, &u, 2);
  return static_cast<float>(h);
}

// ---------------------------------------------------------------------------
// Matrix-core kernel: grid (B*S, nsplit), 512 threads (8 waves), one
// workgroup per CU.
// ---------------------------------------------------------------------------
template <bool HCA, bool SPLIT, bool Q4>
__global__ __launch_bounds__(kThreads) void attn_mfma(AttnArgs a, int nsplit, int chunk_rows) {
  __shared__ __attribute__((aligned(16))) unsigned char tiles[kBufs][kT * kPitch];
  __shared__ __attribute__((aligned(16))) uint16_t pt[2][kH * kPPitch];
  __shared__ __attribute__((aligned(4))) uint8_t vmask[kBufs][kWaves];
  __shared__ float lsum[2][kH];
  __shared__ float mseen[2][kH];
  __shared__ float mref[kH];  // reference of the current pass, per head
  __shared__ int over_flag;
  __shared__ int codes[kMaxChunk];  // resolved candidate codes (HCA: only for a paged cache)
  __shared__ float amax[SPLIT ? 4 : 1][kH];  // split partials: largest |O|/l per PV wave and head
  __shared__ float escale[SPLIT ? kH : 1];   // split partials: the head's exponent e

  const int64_t qi = blockIdx.x;
  const int split = blockIdx.y;
  const int b = int(qi / a.S);
  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int g = lane / 16, c16 = lane % 16;
  const int64_t j_begin = int64_t(split) * chunk_rows;
  // Q (64 KiB) comes in once through the load unit, into the space of tile
  // buffers 2 and 3 (every wave copies 8 head rows; 16-byte chunk c of head
  // h's row sits at chunk c ^ (h % 16), so that the QK waves' reads are
  // conflict-free); the QK waves take their Q^T operands from LDS, and then
  // tiles 2 and 3 follow.  CSA requests Q first of all, so that it lands
  // during the round trip of the position and the selection entries, ahead
  // of the row copies (0.25 us less at a 64K context); HCA requests it
  // beside tiles 0 and 1, whose copies need no selection (Q first measured
  // 0.15 us slower there).
  auto issue_q = [&]() {
    static_assert(kH * kRowBytes <= 2 * kT * kPitch, "Q fits in two tile buffers");
    const uint32_t lds_q = uint32_t(reinterpret_cast<uintptr_t>((lds_void*)&tiles[2][0]));
    const uint16_t* q = static_cast<const uint16_t*>(a.q) + qi * kH * kD;
#pragma unroll
    for (int r = 0; r < kH / kWaves; ++r) {
      const int h = wave * (kH / kWaves) + r;
      copy_row_to_lds(q + h * kD, uint32_t(lane ^ (h % 16)) * 16u, lds_q + uint32_t(h * kRowBytes));
    }
  };
  if constexpr (!HCA) issue_q();
  // CSA: the chunk's selection entries are requested beside the position,
  // as if the window were full (true for every query at or past its
  // window'th token), so that one round trip brings both; a query with a
  // shorter window reads its entries again below
  constexpr int kSpecPer = (kMaxChunk + kThreads - 1) / kThreads;
  int spec[kSpecPer];
  if constexpr (!HCA) {
#pragma unroll
    for (int t = 0; t < kSpecPer; ++t) {
      const int j = tid + t * kThreads;
      const int64_t i = j_begin + j - a.window;
      spec[t] = (j < chunk_rows && i >= 0 && i < a.k) ? a.idx[qi * a.k + i] : -1;
    }
  }
  const Cand c = candidates(a, HCA, qi);
  const int64_t n_cand = c.n_win + c.n_sel;
  const int n_rows = int(j_begin < n_cand ? (n_cand - j_begin < chunk_rows ? n_cand - j_begin : chunk_rows) : 0);
  const int n_tiles = (n_rows + kT - 1) / kT;
  const uint16_t* win = static_cast<const uint16_t*>(a.win) + int64_t(b) * a.Wcap * kD;
  // candidate codes are pool rows when the cache is paged
  const uint16_t* cmp = static_cast<const uint16_t*>(a.cmp) + (a.pt.pages ? 0 : int64_t(b) * a.Ncap * kD);
  // a readable 1 KiB row (the query's first head) stands in for a missing
  // candidate: its score is masked, and its finite values keep 0 * row = 0
  const uint16_t* filler = static_cast<const uint16_t*>(a.q) + qi * kH * kD;

  // Quantised compressed rows (Q4): the load unit copies a row's raw bytes
  // into the start of its tile slot (one copy per row, like a bf16 row), and
  // the wave that copied it turns it into bf16 in place once the copy has
  // landed, just before the barrier that publishes the tile.  Lane l takes
  // channels 8l .. 8l+7.
  const unsigned char* cmp_q =
      static_cast<const unsigned char*>(a.cmp) + (a.pt.pages ? 0 : int64_t(b) * a.Ncap * a.cmp_row_bytes);
  const bool lane_fp4 = 8 * lane < kD - a.rope_dim;
  // E2M1 lanes read the 8-byte aligned pair of code words holding theirs
  const int q_code_off = lane_fp4 ? 8 * (lane / 2) : kv4_code_offset(8 * lane, kD, a.rope_dim);
  const int q_scale_off = kv4_scale_offset(8 * lane, kD, a.rope_dim);
  const int q_lanes = a.cmp_row_bytes / 16;  // lanes that copy a raw row, 16 bytes each
  uint32_t q4mask = 0;  // per tile buffer (4 bits each): the wave's rows that hold raw quantised bytes

  // CSA: resolve the chunk's selections once, so that row copies never wait
  // on a dependent index load
  const bool resolved = !HCA || a.pt.pages != nullptr;  // HCA: contiguous rows need no table
  if (resolved) {
#pragma unroll
    for (int t = 0; t < kSpecPer; ++t) {
      const int j = tid + t * kThreads;
      if (j >= n_rows) continue;
      int code;
      if (!HCA && c.n_win == a.window && j_begin + j >= c.n_win) {
        const int e = spec[t];  // the selection entry of candidate j_begin + j
        code = (e >= 0 && e < a.Ncap) ? (a.pt.pages ? int(paged_row(a.pt, b, e)) : e) : -1;
      } else {
        code = cand_code(a, HCA, c, qi, j_begin + j);
      }
      codes[j] = code;
    }
  }
  if (tid == 0) over_flag = 0;
  if (tid < kH) mref[tid] = sink_ref(a.sink, tid);
  if constexpr (!HCA) wait_vmem<0>();  // Q (and the selection entries) have landed
  __syncthreads();
  const uint32_t lds_tiles = uint32_t(reinterpret_cast<uintptr_t>((lds_void*)&tiles[0][0]));
  // wave w copies rows kCopyRows*w .. +kCopyRows-1 of tile t (always exactly
  // kCopyRows copies, so that the copy count in flight is known) and records
  // which of them exist
  auto issue = [&](int t) {
    const int buf = t % kBufs;
    const int jl = t * kT + wave * kCopyRows + (lane % kCopyRows);
    int code = -1;
    if (jl < n_rows) code = resolved ? codes[jl] : cand_code(a, true, c, qi, j_begin + jl);
    const uint64_t ok = __ballot(code != -1);
    if (lane == 0) vmask[buf][wave] = uint8_t(ok & ((1u << kCopyRows) - 1u));
    const uint32_t dst = lds_tiles + uint32_t(buf * kT * kPitch + wave * kCopyRows * kPitch);
    const uint32_t voff = uint32_t(lane ^ (row_flip(wave * kCopyRows) << 3)) * 16u;  // same for the wave's rows
    uint32_t qm = 0;
#pragma unroll
    for (int u = 0; u < kCopyRows; ++u) {
      const int cu = __builtin_amdgcn_readlane(code, u);
      if (Q4 && cu >= 0) {
        // raw bytes of the quantised row, in order, from the slot's start
        if (lane < q_lanes) copy_row_to_lds(cmp_q + int64_t(cu) * a.cmp_row_bytes, uint32_t(lane) * 16u,
                                            dst + uint32_t(u * kPitch));
        qm |= 1u << u;
      } else {
        const uint16_t* src = cu >= 0 ? cmp + int64_t(cu) * kD : (cu <= -2 ? win + int64_t(-2 - cu) * kD : filler);
        copy_row_to_lds(src, voff, dst + uint32_t(u * kPitch));
      }
    }
    if constexpr (Q4) q4mask = (q4mask & ~(15u << (4 * buf))) | (qm << (4 * buf));
  };
  // Q4: the wave's quantised rows of tile t, turned into bf16 in place (each
  // lane reads its code bytes and scale byte, then writes its 16-byte chunk
  // where a bf16 row copy would have put it; a row's reads all happen before
  // its writes, so the overlap is harmless)
  auto dequant_tile = [&](int t) {
    const int buf = t % kBufs;
    const uint32_t qm = (q4mask >> (4 * buf)) & 15u;
    if (qm == 0) return;
    unsigned char* slot0 = &tiles[buf][0] + wave * kCopyRows * kPitch;
    const int chunk = (lane ^ (row_flip(wave * kCopyRows) << 3)) * 16;
#pragma unroll
    for (int u = 0; u < kCopyRows; ++u) {
      if (!((qm >> u) & 1u)) continue;
      unsigned char* slot = slot0 + u * kPitch;
      uint2 cw = *reinterpret_cast<const uint2*>(slot + q_code_off);
      const uint32_t sb = slot[q_scale_off];
      if (lane_fp4) cw.x = (lane & 1) ? cw.y : cw.x;
      *reinterpret_cast<uint4*>(slot + chunk) = kv4_lane_bf16(cw, sb, lane_fp4);
    }
  };
  // The first min(n_tiles, kBufs) tiles are copied up front (every buffer is
  // free then); afterwards step s copies tile s+2 into the buffer that tile
  // s-2 left.  Top of step s: tile s has landed (only later tiles' copies may
  // be in flight), then the barrier publishes it.
  auto prologue = [&]() {
    for (int t = 0; t < n_tiles && t < kBufs; ++t) issue(t);
  };
  auto step_sync = [&](int s) {
    const int hi = s + 2 > kBufs ? s + 2 : kBufs;
    const int later = (n_tiles < hi ? n_tiles : hi) - (s + 1);  // tiles issued after tile s
    if (later >= 3) wait_vmem<3 * kCopyRows>();
    else if (later == 2) wait_vmem<2 * kCopyRows>();
    else if (later == 1) wait_vmem<kCopyRows>();
    else wait_vmem<0>();
    if constexpr (Q4) {
      if (s < n_tiles) dequant_tile(s);  // this wave's copies of tile s have landed
    }
    __syncthreads();
    if (s + 2 >= kBufs && s + 2 < n_tiles) issue(s + 2);
  };
  const float qk_scale = a.scale * kLog2e;

  if constexpr (HCA) {
    issue_q();
    for (int t = 0; t < n_tiles && t < 2; ++t) issue(t);
    if (n_tiles >= 2) wait_vmem<2 * kCopyRows>();  // Q has landed; tiles 0 and 1 may still be in flight
    else if (n_tiles == 1) wait_vmem<kCopyRows>();
    else wait_vmem<0>();
    __syncthreads();
  } else {
    for (int t = 0; t < n_tiles && t < 2; ++t) issue(t);
  }
  // once Q is in the QK waves' registers, buffers 2 and 3 take tiles 2 and 3
  auto issue_rest = [&]() {
    __syncthreads();
    for (int t = 2; t < n_tiles && t < kBufs; ++t) issue(t);
  };

  if (wave < 4) {
    // ===================== QK waves =====================
    const int hh = wave & 1, rr = wave >> 1;  // heads hh*32.., rows rr*16.. of a tile
    bf16x8 qb[2][16];  // Q^T: Q[hh*32 + ht*16 + c16][ks*32 + g*8 .. +7]
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) {
      const unsigned char* qrow = &tiles[2][0] + (hh * 32 + ht * 16 + c16) * kRowBytes;
#pragma unroll
      for (int ks = 0; ks < 16; ++ks)
        qb[ht][ks] = as_bf16x8(*reinterpret_cast<const uint4*>(qrow + (((ks * 4 + g) ^ c16) << 4)));
    }
    issue_rest();
    // K chunk ks*4 + g of row rr*16 + c16 sits 128 B further (K-steps with
    // bit 1 clear) or nearer (bit 1 set) when the row is flipped
    const int k_base = (rr * 16 + c16) * kPitch + g * 16;
    const int k_off0 = k_base + row_flip(c16) * 128, k_off1 = k_base - row_flip(c16) * 128;
    float m_ref[2];
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) m_ref[ht] = sink_ref(a.sink, hh * 32 + ht * 16 + c16);
    for (int pass = 0; pass < 2; ++pass) {
      float l_run[2], m_run[2];
      bool over = false;
#pragma unroll
      for (int ht = 0; ht < 2; ++ht) {
        const float s2 = a.sink[hh * 32 + ht * 16 + c16] * kLog2e;
        l_run[ht] = (!SPLIT && rr == 0 && g == 0) ? fast_exp2(s2 - m_ref[ht]) : 0.f;
        m_run[ht] = -INFINITY;
      }
      if (pass > 0) prologue();
      for (int s = 0; s <= n_tiles; ++s) {
        step_sync(s);
        if (s == n_tiles) break;
        const unsigned char* tile = tiles[s % kBufs];
        const uint32_t okm = *reinterpret_cast<const uint32_t*>(&vmask[s % kBufs][rr * 4]);  // rows rr*16 + 4*w' + u
        // ---- S^T = K . Q^T, K operands kAheadK K-steps ahead
        floatx4 st[2] = {floatx4{0.f, 0.f, 0.f, 0.f}, floatx4{0.f, 0.f, 0.f, 0.f}};
        bf16x8 kr[kAheadK + 1];
#pragma unroll
        for (int ks = 0; ks < kAheadK; ++ks)
          kr[ks] = as_bf16x8(*reinterpret_cast<const uint4*>(tile + ((ks & 2) ? k_off1 : k_off0) + ks * 64));
#pragma unroll
        for (int ks = 0; ks < 16; ++ks) {
          if (ks + kAheadK < 16)
            kr[(ks + kAheadK) % (kAheadK + 1)] = as_bf16x8(*reinterpret_cast<const uint4*>(
                tile + (((ks + kAheadK) & 2) ? k_off1 : k_off0) + (ks + kAheadK) * 64));
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int ht = 0; ht < 2; ++ht)
            st[ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kr[ks % (kAheadK + 1)], qb[ht][ks], st[ht], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
        // ---- P = exp2(S - m): rows rr*16 + g*4 + i, head hh*32 + ht*16 + c16
        uint16_t* pw = &pt[s & 1][0];
#pragma unroll
        for (int ht = 0; ht < 2; ++ht) {
          float p[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const bool ok = (okm >> (8 * g + i)) & 1u;  // byte g of okm = wave rr*4 + g, bit i
            const float sv = ok ? st[ht][i] * qk_scale : -INFINITY;
            m_run[ht] = fmaxf(m_run[ht], sv);
            p[i] = fast_exp2(sv - m_ref[ht]);
          }
          over = over || (m_run[ht] > m_ref[ht] + kHeadroom);
          l_run[ht] += (p[0] + p[1]) + (p[2] + p[3]);
          *reinterpret_cast<uint2*>(&pw[(hh * 32 + ht * 16 + c16) * kPPitch + rr * 16 + g * 4]) =
              uint2{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])};
        }
      }
      // ---- per-head sums and maxima of this wave's rows
#pragma unroll
      for (int ht = 0; ht < 2; ++ht) {
        const float l = sum_rows4(l_run[ht]);
        const float m = max_rows4(m_run[ht]);
        if (g == 0) {
          lsum[rr][hh * 32 + ht * 16 + c16] = l;
          mseen[rr][hh * 32 + ht * 16 + c16] = m;
        }
      }
      if (__any(over) && lane == 0) over_flag = 1;
      __syncthreads();
      if (over_flag == 0) break;
#pragma unroll
      for (int ht = 0; ht < 2; ++ht) {
        const int h = hh * 32 + ht * 16 + c16;
        m_ref[ht] = fmaxf(sink_ref(a.sink, h), fmaxf(mseen[0][h], mseen[1][h]));
        if (rr == 0 && g == 0) mref[h] = m_ref[ht];
      }
      __syncthreads();  // every wave has read the flag and the maxima
      if (tid == 0) over_flag = 0;
    }
    if constexpr (SPLIT) {
      __syncthreads();  // the PV waves' largest values
      if (tid < kH) {
        const float am = fmaxf(fmaxf(amax[0][tid], amax[1][tid]), fmaxf(amax[2][tid], amax[3][tid]));
        // am < 2^ex; e keeps am * 2^-e below 2^15
        const int ex = am > 0.f ? int((__float_as_uint(am) >> 23) & 0xffu) - 126 : 0;
        const int e = ex > 15 ? ex - 15 : 0;
        escale[tid] = float(e);
        float4* ml = reinterpret_cast<float4*>(partial_ml(a, nsplit));
        ml[(qi * nsplit + split) * kH + tid] = float4{mref[tid], lsum[0][tid] + lsum[1][tid], float(e), 0.f};
      }
      __syncthreads();  // the exponents
    }
  } else {
    // ===================== PV waves =====================
    const int pv = wave - 4;  // dims pv*128 .. +128
    issue_rest();
    // V^T operand: rows g*8 + h*4 + c16/4 (h = half of the 8-row K-slice),
    // dims pv*128 + dt*16 + 4*(c16 % 4) .. +3; a flipped row (bit 2 = h,
    // bit 3 = g & 1) holds the chunk 128 B further (dt < 4) or nearer (dt >= 4)
    const int v_base = (g * 8 + (c16 >> 2)) * kPitch + pv * 256 + (((c16 >> 1) & 1) << 4) + ((c16 & 1) << 3);
    const int f_lo = (g & 1) * 128, f_hi = ((g & 1) ^ 1) * 128;
    const int v_lo0 = v_base + f_lo, v_lo1 = v_base - f_lo;
    const int v_hi0 = v_base + 4 * kPitch + f_hi, v_hi1 = v_base + 4 * kPitch - f_hi;
    floatx4 acc[8][4];  // O^T[dims pv*128 + dt*16 + g*4 + i][head ht*16 + c16]
    for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int ht = 0; ht < 4; ++ht) acc[dt][ht] = floatx4{0.f, 0.f, 0.f, 0.f};
      if (pass > 0) prologue();
      for (int s = 0; s <= n_tiles; ++s) {
        step_sync(s);
        if (s == 0) continue;
        const unsigned char* tile = tiles[(s - 1) % kBufs];
        const uint16_t* pr = &pt[(s - 1) & 1][0];
        bf16x8 pb[4];  // P^T[rows g*8 .. +7][head ht*16 + c16]
#pragma unroll
        for (int ht = 0; ht < 4; ++ht)
          pb[ht] = as_bf16x8(*reinterpret_cast<const uint4*>(&pr[(ht * 16 + c16) * kPPitch + g * 8]));
        bf16x8 vr[kAheadV + 1];
        auto vload = [&](int dt, bf16x8& dst) {
          const uint2 lo = lds_read_tr16(tile + ((dt & 4) ? v_lo1 : v_lo0) + dt * 32);
          const uint2 hi = lds_read_tr16(tile + ((dt & 4) ? v_hi1 : v_hi0) + dt * 32);
          dst = as_bf16x8(uint4{lo.x, lo.y, hi.x, hi.y});
        };
#pragma unroll
        for (int dt = 0; dt < kAheadV; ++dt) vload(dt, vr[dt]);
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          if (dt + kAheadV < 8) vload(dt + kAheadV, vr[(dt + kAheadV) % (kAheadV + 1)]);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int ht = 0; ht < 4; ++ht)
            acc[dt][ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vr[dt % (kAheadV + 1)], pb[ht], acc[dt][ht], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      __syncthreads();  // the QK waves' sums, maxima and overflow flag
      if (over_flag == 0) break;
      __syncthreads();
    }
    float L[4];
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) L[ht] = lsum[0][ht * 16 + c16] + lsum[1][ht * 16 + c16];
    if constexpr (!SPLIT) {
      const int rope0 = kD - a.rope_dim;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const int d0 = pv * 128 + dt * 16 + g * 4;
        float cs[2] = {1.f, 1.f}, sn[2] = {0.f, 0.f};
        const bool rot = d0 >= rope0 && c.p >= 0;
        if (rot) {
#pragma unroll
          for (int u = 0; u < 2; ++u) rope_cos_sin(c.p, (d0 + 2 * u - rope0) / 2, a.rope_dim, a.rope_log2_base, &cs[u], &sn[u]);
        }
#pragma unroll
        for (int ht = 0; ht < 4; ++ht) {
          const float inv_l = 1.f / L[ht];
          float o[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) o[i] = acc[dt][ht][i] * inv_l;
          if (rot) {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
              const float x0 = o[2 * u], x1 = o[2 * u + 1];
              o[2 * u] = x0 * cs[u] + x1 * sn[u];
              o[2 * u + 1] = x1 * cs[u] - x0 * sn[u];
            }
          }
          const int64_t off = (qi * kH + ht * 16 + c16) * kD + d0;
          if (a.out_dtype == CSA_BF16) {
            *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + off) =
                uint2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
          } else {
            *reinterpret_cast<float4*>(static_cast<float*>(a.out) + off) = float4{o[0], o[1], o[2], o[3]};
          }
        }
      }
    } else {
      // O / l per head, its largest magnitude over this wave's dims to LDS
      float inv[4];
#pragma unroll
      for (int ht = 0; ht < 4; ++ht) {
        inv[ht] = L[ht] > 0.f ? 1.f / L[ht] : 0.f;
        float m = 0.f;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
#pragma unroll
          for (int i = 0; i < 4; ++i) m = fmaxf(m, fabsf(acc[dt][ht][i]));
        m = max_rows4(m);
        if (g == 0) amax[pv][ht * 16 + c16] = m * inv[ht];
      }
      __syncthreads();  // largest values in
      __syncthreads();  // exponents out
      uint4* ws_o = static_cast<uint4*>(a.ws) + (qi * nsplit + split) * kPartialVecs;
#pragma unroll
      for (int ht = 0; ht < 4; ++ht) {
        const float f = inv[ht] * __uint_as_float(uint32_t(127 - int(escale[ht * 16 + c16])) << 23);  // inv * 2^-e
#pragma unroll
        for (int dp = 0; dp < 4; ++dp) {
          const floatx4 x = acc[2 * dp][ht], y = acc[2 * dp + 1][ht];
          ws_o[partial_block(pv, dp, ht) * kWave + lane] =
              uint4{pack_f16x2(x[0] * f, x[1] * f), pack_f16x2(x[2] * f, x[3] * f), pack_f16x2(y[0] * f, y[1] * f),
                    pack_f16x2(y[2] * f, y[3] * f)};
        }
      }
    }
  }
}

// Merge the splits of one query with the sink, inverse RoPE, store.  grid
// (B*S, 64): workgroup y = (v, dp, ht) takes partial block y of every split;
// 256 threads, wave w sums the splits w, w+4, ... (BATCH of its loads in
// flight at once), the four sums meet in LDS.  A small BATCH for few splits
// keeps the registers low enough for eight workgroups per CU, so that large
// batches of queries (64 workgroups each) merge in one round.
template <int BATCH>
__global__ __launch_bounds__(256) void attn_combine(AttnArgs a, int nsplit) {
  __shared__ __attribute__((aligned(16))) float part[4][kWave][8];
  // per split and head of the block: reference, sum, log2 of the stored scale
  // (3 x nsplit x 16 floats of dynamic LDS)
  extern __shared__ float rec[];
  float (*sm)[16] = reinterpret_cast<float (*)[16]>(rec);
  float (*sl)[16] = reinterpret_cast<float (*)[16]>(rec + nsplit * 16);
  float (*se)[16] = reinterpret_cast<float (*)[16]>(rec + 2 * nsplit * 16);
  const int64_t qi = blockIdx.x;
  const int blk = blockIdx.y;
  const int v = blk / 16, dp = (blk / 4) % 4, ht = blk % 4;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int g = lane / 16, c16 = lane % 16;
  const int h = ht * 16 + c16;
  const uint4* ws_o = static_cast<const uint4*>(a.ws) + qi * nsplit * kPartialVecs + blk * kWave + lane;
  // this wave's partials (splits wave, wave + 4, ...) are requested first:
  // they need no record, so their latency overlaps the records' own
  constexpr int kBatch = BATCH;  // splits per wave held at once
  uint4 u[kBatch];
#pragma unroll
  for (int j = 0; j < kBatch; ++j) {
    const int sp = wave + 4 * j;
    if (sp < nsplit) u[j] = ws_o[int64_t(sp) * kPartialVecs];
  }
  // every split's record for the 16 heads into LDS, four loads in flight per thread
  {
    const float4* ml = reinterpret_cast<const float4*>(partial_ml(a, nsplit));
    const int n = nsplit * 16;
    for (int i0 = tid; i0 < n; i0 += 4 * 256) {
      float4 w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i = i0 + j * 256;
        if (i < n) w[j] = ml[(qi * nsplit + i / 16) * kH + ht * 16 + i % 16];
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i = i0 + j * 256;
        if (i < n) {
          sm[i / 16][i % 16] = w[j].x;
          sl[i / 16][i % 16] = w[j].y;
          se[i / 16][i % 16] = w[j].z;
        }
      }
    }
  }
  __syncthreads();
  // the head's largest reference and its sum: lanes g = 0..3 of a head take
  // the splits s = g mod 4
  const float sink2 = a.sink[h] * kLog2e;
  float mx = sink2;
  for (int s = g; s < nsplit; s += 4) mx = fmaxf(mx, sm[s][c16]);
  mx = max_rows4(mx);
  float l = 0.f;
  for (int s = g; s < nsplit; s += 4) l += sl[s][c16] * fast_exp2(sm[s][c16] - mx);
  const float L = sum_rows4(l) + fast_exp2(sink2 - mx);

  float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int s0 = wave; s0 < nsplit; s0 += 4 * kBatch) {
    if (s0 != wave) {  // more than kBatch splits per wave
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const int sp = s0 + 4 * j;
        if (sp < nsplit) u[j] = ws_o[int64_t(sp) * kPartialVecs];
      }
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int sp = s0 + 4 * j;
      if (sp < nsplit) {
        const float fj = sl[sp][c16] * fast_exp2(sm[sp][c16] + se[sp][c16] - mx);  // l_s 2^(m_s - mx + e_s)
        o[0] += fj * f16_lo(u[j].x); o[1] += fj * f16_hi(u[j].x); o[2] += fj * f16_lo(u[j].y); o[3] += fj * f16_hi(u[j].y);
        o[4] += fj * f16_lo(u[j].z); o[5] += fj * f16_hi(u[j].z); o[6] += fj * f16_lo(u[j].w); o[7] += fj * f16_hi(u[j].w);
      }
    }
  }
  *reinterpret_cast<float4*>(&part[wave][lane][0]) = float4{o[0], o[1], o[2], o[3]};
  *reinterpret_cast<float4*>(&part[wave][lane][4]) = float4{o[4], o[5], o[6], o[7]};
  __syncthreads();
  if (wave != 0) return;
  const float inv = 1.f / L;
  float y[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = ((part[0][lane][i] + part[1][lane][i]) + (part[2][lane][i] + part[3][lane][i])) * inv;
  const int rope0 = kD - a.rope_dim;
  const int p = a.pos[qi];
#pragma unroll
  for (int half = 0; half < 2; ++half) {  // dims 128v + 32dp + 16 half + 4g + 0..3
    const int d0 = v * 128 + dp * 32 + half * 16 + g * 4;
    float* x = &y[4 * half];
    if (d0 >= rope0 && p >= 0) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        float cs, sn;
        rope_cos_sin(p, (d0 + 2 * u - rope0) / 2, a.rope_dim, a.rope_log2_base, &cs, &sn);
        const float x0 = x[2 * u], x1 = x[2 * u + 1];
        x[2 * u] = x0 * cs + x1 * sn;
        x[2 * u + 1] = x1 * cs - x0 * sn;
      }
    }
    const int64_t off = (qi * kH + h) * kD + d0;
    if (a.out_dtype == CSA_BF16) {
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + off) = uint2{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
    } else {
      *reinterpret_cast<float4*>(static_cast<float*>(a.out) + off) = float4{x[0], x[1], x[2], x[3]};
    }
  }
}

// ---------------------------------------------------------------------------
// Persistent matrix-core kernel for many queries without splits (prefill).
// Grid G (about one workgroup per CU), 512 threads.  Workgroup x runs the
// queries x, x + G, x + 2G, ... (at most kPMaxQ) as ONE stream of 32-row
// tiles through the same warp-specialised pipeline as attn_mfma, so that row
// copies and selection loads run ahead across query boundaries, the QK waves
// load the next query's Q^T while the PV waves still work on the previous
// query, and no query pays a pipeline fill or drain of its own.
//   * PV waves issue every copy: wave 4+v copies rows 8v..8v+7 of each tile,
//     and wave 4 also copies the next query's selection list into LDS when
//     the copies enter a query (two list buffers, by query parity);
//   * the QK waves start a query's sums at its first tile and hand them (and
//     an overflow flag) to the PV waves at its last tile, by query parity;
//   * the PV waves zero O at a query's first tile and normalise, rotate and
//     store it in the step that consumes its last tile.
// The sink reference of attn_mfma is kept; a query whose scores exceed it by
// more than the headroom is flagged in redo[qi] and recomputed exactly by
// attn_redo (never for ordinary data).
// ---------------------------------------------------------------------------
constexpr int kPMaxQ = 64;               // queries per workgroup
constexpr int kPCopyRows = kT / 8;       // rows each wave copies per tile
constexpr int kPMaxSel = 1024;           // CSA selections of a query staged in LDS
constexpr int kPersistMinQueries = 512;  // fewer queries take attn_mfma
constexpr int kEpiStores = 8 * 4;        // output stores per PV lane when a query ends (one per dim x head tile)

// One selection-list copy HBM -> LDS: lane l moves the dword at base + voff to
// LDS address lds + 4 l (wait states as in copy_row_to_lds).
__device__ __forceinline__ void copy_dwords_to_lds(const void* base, uint32_t voff, uint32_t lds) {
  const uint64_t r = reinterpret_cast<uint64_t>(base);
  const uint64_t su = uint64_t(uint32_t(__builtin_amdgcn_readfirstlane(uint32_t(r)))) |
                      (uint64_t(uint32_t(__builtin_amdgcn_readfirstlane(uint32_t(r >> 32)))) << 32);
  asm volatile("s_nop 4\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(su), "{m0}"(lds) : "memory");
}

template <bool HCA>
__global__ __launch_bounds__(kThreads) void attn_persist(AttnArgs a, int* redo) {
  __shared__ __attribute__((aligned(16))) unsigned char tiles[kBufs][kT * kPitch];
  __shared__ __attribute__((aligned(16))) uint16_t pt[2][kH * kPPitch];
  __shared__ __attribute__((aligned(4))) uint8_t vmask[kBufs][8];  // [tile buffer][wave]: rows 4w + bit
  __shared__ __attribute__((aligned(16))) int sel[2][HCA ? 1 : kPMaxSel];
  __shared__ float lsum[2][2][kH];  // [query parity][QK row half][head]
  __shared__ int ovf[2][4];         // [query parity][QK wave]
  __shared__ int qpos[kPMaxQ];

  const int G = gridDim.x;
  const int x = blockIdx.x;
  const int nq = a.B * a.S;
  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int g = lane / 16, c16 = lane % 16;
  const int nqb = (nq - x + G - 1) / G;  // this workgroup's queries (x < nq, nqb <= kPMaxQ)
  if (tid < nqb) qpos[tid] = a.pos[x + tid * G];
  __syncthreads();

  // candidate layout of the workgroup's query k
  struct Query {
    int k, qi, b, p, n_win, n_sel, s0, nt;
  };
  auto query = [&](int k) -> Query {
    Query c;
    c.k = k;
    c.qi = x + k * G;
    c.b = c.qi / a.S;
    c.p = __builtin_amdgcn_readfirstlane(qpos[k]);
    c.n_win = 0;
    c.n_sel = 0;
    c.s0 = 0;
    if (c.p >= 0) {
      c.n_win = c.p + 1 < a.window ? c.p + 1 : a.window;
      c.s0 = int(uint32_t(c.p - c.n_win + 1) % uint32_t(a.Wcap));
      if (HCA) {
        const int nv = int((int64_t(c.p) + 1) / a.ratio);
        c.n_sel = nv < a.Ncap ? nv : a.Ncap;
      } else {
        c.n_sel = a.k;
      }
    }
    const int64_t n = int64_t(c.n_win) + c.n_sel;
    c.nt = n > 0 ? int((n + kT - 1) / kT) : 1;  // a query with no candidates runs one masked tile
    return c;
  };
  // a position in the stream: tile t of query c
  struct Cur {
    Query c;
    int t;
  };
  auto advance = [&](Cur& u) {
    if (++u.t == u.c.nt) {
      u.t = 0;
      if (u.c.k + 1 < nqb) u.c = query(u.c.k + 1);
      else u.c.k = nqb;
    }
  };
  int total = 0;
  for (int k = 0; k < nqb; ++k) total += query(k).nt;
  const Cur first{query(0), 0};

  const uint32_t lds_tiles = uint32_t(reinterpret_cast<uintptr_t>((lds_void*)&tiles[0][0]));
  const uint32_t lds_sel = uint32_t(reinterpret_cast<uintptr_t>((lds_void*)&sel[0][0]));
  // selection list of query k -> sel[k & 1] (wave 4 only)
  auto copy_sel = [&](int k) {
    const int* src = a.idx + int64_t(x + k * G) * a.k;
    const uint32_t dst = lds_sel + uint32_t((k & 1) * kPMaxSel * 4);
    for (int m = 0; m * kWave < a.k; ++m) {
      const int i = m * kWave + lane;
      copy_dwords_to_lds(src, uint32_t(i < a.k ? i : 0) * 4u, dst + uint32_t(m * kWave * 4));
    }
  };
  // copies of stream tile u (tile u.t of query u.c) into buffer u % kBufs:
  // wave w copies rows 4w .. 4w+3 (every wave, so that no wave group stalls
  // on all of a tile's copies)
  auto issue = [&](const Cur& cu, int u) {
    if (!HCA && wave == 4 && cu.t == 0 && cu.c.k + 1 < nqb) copy_sel(cu.c.k + 1);  // lands before cu's next query
    const int buf = u % kBufs;
    const int j = cu.t * kT + wave * kPCopyRows + (lane % kPCopyRows);
    int code = -1;  // >= 0 compressed entry, <= -2 window ring slot, -1 none
    if (j < cu.c.n_win) {
      const int slot = cu.c.s0 + j;
      code = -2 - (slot >= a.Wcap ? slot - a.Wcap : slot);
    } else if (j - cu.c.n_win < cu.c.n_sel) {
      const int i = j - cu.c.n_win;
      if (HCA) {
        code = i;
      } else {
        const int e = sel[cu.c.k & 1][i];
        code = (e >= 0 && e < a.Ncap) ? e : -1;
      }
    }
    const uint64_t ok = __ballot(code != -1);
    if (lane == 0) vmask[buf][wave] = uint8_t(ok & 0xfu);
    const uint16_t* win = static_cast<const uint16_t*>(a.win) + int64_t(cu.c.b) * a.Wcap * kD;
    const uint16_t* cmp = static_cast<const uint16_t*>(a.cmp) + int64_t(cu.c.b) * a.Ncap * kD;
    // the query's first head row stands in for a missing candidate (masked, finite)
    const uint16_t* filler = static_cast<const uint16_t*>(a.q) + int64_t(cu.c.qi) * kH * kD;
    const uint32_t dst = lds_tiles + uint32_t(buf * kT * kPitch + wave * kPCopyRows * kPitch);
    // the wave's four rows share one chunk flip (row_flip)
    const uint32_t voff = uint32_t(lane ^ (row_flip(wave * kPCopyRows) << 3)) * 16u;
    // lane r forms row r's address; each copy reads it back as a scalar pair
    const uint16_t* src = code >= 0 ? cmp + int64_t(code) * kD : (code <= -2 ? win + int64_t(-2 - code) * kD : filler);
    const uint64_t sa = reinterpret_cast<uint64_t>(src);
#pragma unroll
    for (int r = 0; r < kPCopyRows; ++r) {
      const uint64_t ra = uint64_t(uint32_t(__builtin_amdgcn_readlane(uint32_t(sa), r))) |
                          (uint64_t(uint32_t(__builtin_amdgcn_readlane(uint32_t(sa >> 32), r))) << 32);
      copy_row_to_lds(reinterpret_cast<const void*>(ra), voff, dst + uint32_t(r * kPitch));
    }
  };
  const float qk_scale = a.scale * kLog2e;

  if (wave < 4) {
    // ===================== QK waves =====================
    const int hh = wave & 1, rr = wave >> 1;
    bf16x8 qb[2][16];
    auto load_q = [&](int qi) {
#pragma unroll
      for (int ht = 0; ht < 2; ++ht) {
        const uint16_t* q =
            static_cast<const uint16_t*>(a.q) + (int64_t(qi) * kH + hh * 32 + ht * 16 + c16) * kD + g * 8;
#pragma unroll
        for (int ks = 0; ks < 16; ++ks) qb[ht][ks] = as_bf16x8(*reinterpret_cast<const uint4*>(q + ks * 32));
      }
    };
    load_q(first.c.qi);
    wait_vmem<0>();  // Q^T in registers before any copy is issued
    // prologue, in step with the PV waves: first selection list, tile 0,
    // second selection list, tile 1
    Cur ci = first;
    __syncthreads();
    issue(ci, 0);
    advance(ci);
    __syncthreads();
    if (total > 1) {
      issue(ci, 1);
      advance(ci);
    }
    const int k_base = (rr * 16 + c16) * kPitch + g * 16;
    const int k_off0 = k_base + row_flip(c16) * 128, k_off1 = k_base - row_flip(c16) * 128;
    float m_ref[2], l_sink[2];
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) {
      const int h = hh * 32 + ht * 16 + c16;
      m_ref[ht] = sink_ref(a.sink, h);
      l_sink[ht] = (rr == 0 && g == 0) ? fast_exp2(a.sink[h] * kLog2e - m_ref[ht]) : 0.f;
    }
    float l_run[2] = {0.f, 0.f}, m_run[2] = {-INFINITY, -INFINITY};
    bool over = false;
    Cur cq = first;
    for (int s = 0; s <= total; ++s) {
      // this wave's copies of tile s have landed (only tile s+1's may still fly)
      if (s + 1 < total) wait_vmem<kPCopyRows>();
      else wait_vmem<0>();
      __syncthreads();
      if (s == total) break;
      if (cq.t == 0) {
#pragma unroll
        for (int ht = 0; ht < 2; ++ht) {
          l_run[ht] = l_sink[ht];
          m_run[ht] = -INFINITY;
        }
        over = false;
      }
      const unsigned char* tile = tiles[s % kBufs];
      // rows rr*16 + bit: the nibbles of waves 4rr .. 4rr+3
      const uint32_t w4 = *reinterpret_cast<const uint32_t*>(&vmask[s % kBufs][rr * 4]);
      const uint32_t okm = (w4 & 0xfu) | ((w4 >> 4) & 0xf0u) | ((w4 >> 8) & 0xf00u) | ((w4 >> 12) & 0xf000u);
      floatx4 st[2] = {floatx4{0.f, 0.f, 0.f, 0.f}, floatx4{0.f, 0.f, 0.f, 0.f}};
      bf16x8 kr[kAheadK + 1];
#pragma unroll
      for (int ks = 0; ks < kAheadK; ++ks)
        kr[ks] = as_bf16x8(*reinterpret_cast<const uint4*>(tile + ((ks & 2) ? k_off1 : k_off0) + ks * 64));
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) {
        if (ks + kAheadK < 16)
          kr[(ks + kAheadK) % (kAheadK + 1)] = as_bf16x8(*reinterpret_cast<const uint4*>(
              tile + (((ks + kAheadK) & 2) ? k_off1 : k_off0) + (ks + kAheadK) * 64));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ht = 0; ht < 2; ++ht)
          st[ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kr[ks % (kAheadK + 1)], qb[ht][ks], st[ht], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      const bool last = cq.t == cq.c.nt - 1;
      if (last && cq.c.k + 1 < nqb) {
        // the next query's Q^T, completed here (once per query): the copies
        // issued below then never hold up the next step's products
        load_q(cq.c.qi + G);
        wait_vmem<0>();
      }
      if (s + 2 < total) {
        issue(ci, s + 2);
        advance(ci);
      }
      uint16_t* pw_t = &pt[s & 1][0];
#pragma unroll
      for (int ht = 0; ht < 2; ++ht) {
        float p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool ok = (okm >> (4 * g + i)) & 1u;
          const float sv = ok ? st[ht][i] * qk_scale : -INFINITY;
          m_run[ht] = fmaxf(m_run[ht], sv);
          p[i] = fast_exp2(sv - m_ref[ht]);
        }
        over = over || (m_run[ht] > m_ref[ht] + kHeadroom);
        l_run[ht] += (p[0] + p[1]) + (p[2] + p[3]);
        *reinterpret_cast<uint2*>(&pw_t[(hh * 32 + ht * 16 + c16) * kPPitch + rr * 16 + g * 4]) =
            uint2{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])};
      }
      if (last) {
        const int par = cq.c.k & 1;
#pragma unroll
        for (int ht = 0; ht < 2; ++ht) {
          const float l = sum_rows4(l_run[ht]);
          if (g == 0) lsum[par][rr][hh * 32 + ht * 16 + c16] = l;
        }
        const bool any_over = __any(over);
        if (lane == 0) ovf[par][wave] = any_over ? 1 : 0;
      }
      advance(cq);
    }
  } else {
    // ===================== PV waves =====================
    // prologue: query 0's selection list, then tiles 0 and 1 (tile 0 copies
    // query 1's list first)
    Cur ci = first;
    if (!HCA && wave == 4) copy_sel(0);
    wait_vmem<0>();
    __syncthreads();
    issue(ci, 0);
    advance(ci);
    wait_vmem<kPCopyRows>();  // query 1's list has landed, tile 0 may still be in flight
    __syncthreads();
    if (total > 1) {
      issue(ci, 1);
      advance(ci);
    }
    const int pw = wave - 4;  // PV wave index: dims 128 pw .. 128 pw + 127
    const int v_base = (g * 8 + (c16 >> 2)) * kPitch + pw * 256 + (((c16 >> 1) & 1) << 4) + ((c16 & 1) << 3);
    const int f_lo = (g & 1) * 128, f_hi = ((g & 1) ^ 1) * 128;
    const int v_lo0 = v_base + f_lo, v_lo1 = v_base - f_lo;
    const int v_hi0 = v_base + 4 * kPitch + f_hi, v_hi1 = v_base + 4 * kPitch - f_hi;
    const int rope0 = kD - a.rope_dim;
    floatx4 acc[8][4];
    Cur cp = first;
    bool stored = false;  // the previous step stored a query's output (kEpiStores stores per lane)
    for (int s = 0; s <= total; ++s) {
      // tile s has landed; only tile s+1's copies and the output stores that
      // followed them may still be in flight
      if (s + 1 < total) {
        if (stored) wait_vmem<kPCopyRows + kEpiStores>();
        else wait_vmem<kPCopyRows>();
      } else {
        wait_vmem<0>();
      }
      __syncthreads();
      stored = false;
      if (s + 2 < total) {
        issue(ci, s + 2);
        advance(ci);
      }
      if (s == 0) continue;
      if (cp.t == 0) {
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
#pragma unroll
          for (int ht = 0; ht < 4; ++ht) acc[dt][ht] = floatx4{0.f, 0.f, 0.f, 0.f};
      }
      const unsigned char* tile = tiles[(s - 1) % kBufs];
      const uint16_t* pr = &pt[(s - 1) & 1][0];
      bf16x8 pb[4];
#pragma unroll
      for (int ht = 0; ht < 4; ++ht)
        pb[ht] = as_bf16x8(*reinterpret_cast<const uint4*>(&pr[(ht * 16 + c16) * kPPitch + g * 8]));
      bf16x8 vr[kAheadV + 1];
      auto vload = [&](int dt, bf16x8& dst) {
        const uint2 lo = lds_read_tr16(tile + ((dt & 4) ? v_lo1 : v_lo0) + dt * 32);
        const uint2 hi = lds_read_tr16(tile + ((dt & 4) ? v_hi1 : v_hi0) + dt * 32);
        dst = as_bf16x8(uint4{lo.x, lo.y, hi.x, hi.y});
      };
#pragma unroll
      for (int dt = 0; dt < kAheadV; ++dt) vload(dt, vr[dt]);
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        if (dt + kAheadV < 8) vload(dt + kAheadV, vr[(dt + kAheadV) % (kAheadV + 1)]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ht = 0; ht < 4; ++ht)
          acc[dt][ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vr[dt % (kAheadV + 1)], pb[ht], acc[dt][ht], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (cp.t == cp.c.nt - 1) {
        // the query's last tile: O / sum, inverse RoPE, store
        const int par = cp.c.k & 1;
        const int p = cp.c.p;
        float inv_l[4];
#pragma unroll
        for (int ht = 0; ht < 4; ++ht) inv_l[ht] = 1.f / (lsum[par][0][ht * 16 + c16] + lsum[par][1][ht * 16 + c16]);
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          const int d0 = pw * 128 + dt * 16 + g * 4;
          float cs[2] = {1.f, 1.f}, sn[2] = {0.f, 0.f};
          const bool rot = d0 >= rope0 && p >= 0;
          if (rot) {
#pragma unroll
            for (int u = 0; u < 2; ++u) rope_cos_sin(p, (d0 + 2 * u - rope0) / 2, a.rope_dim, a.rope_log2_base, &cs[u], &sn[u]);
          }
#pragma unroll
          for (int ht = 0; ht < 4; ++ht) {
            float o[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = acc[dt][ht][i] * inv_l[ht];
            if (rot) {
#pragma unroll
              for (int u = 0; u < 2; ++u) {
                const float x0 = o[2 * u], x1 = o[2 * u + 1];
                o[2 * u] = x0 * cs[u] + x1 * sn[u];
                o[2 * u + 1] = x1 * cs[u] - x0 * sn[u];
              }
            }
            const int64_t off = (int64_t(cp.c.qi) * kH + ht * 16 + c16) * kD + d0;
            if (a.out_dtype == CSA_BF16) {
              *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + off) =
                  uint2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
            } else {
              *reinterpret_cast<float4*>(static_cast<float*>(a.out) + off) = float4{o[0], o[1], o[2], o[3]};
            }
          }
        }
        if (pw == 0 && lane == 0) redo[cp.c.qi] = (ovf[par][0] | ovf[par][1] | ovf[par][2] | ovf[par][3]) ? 1 : 0;
        stored = true;
      }
      advance(cp);
    }
  }
}

// ---------------------------------------------------------------------------
// Vector-ALU path for other shapes: one wave per (query, head), online
// softmax over the candidates with the exact running maximum, D <= 1024.
// ---------------------------------------------------------------------------
template <bool HCA>
// (a is taken by value: a reference to the kernel argument made the compiler
// spill the row pointers to the stack and load rows through flat addresses)
__device__ __forceinline__ void attn_head(const AttnArgs a, int64_t qi, int h, float* obuf) {
  const int lane = threadIdx.x;
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
    const bool q4 = !fw && a.cmp_q4;  // a quantised compressed row: row index off / D
    const unsigned char* qrow = static_cast<const unsigned char*>(a.cmp) + (off / D) * a.cmp_row_bytes;
    float rowv[kMaxPer];
    float dot = 0.f;
#pragma unroll
    for (int i = 0; i < kMaxPer; ++i) {
      const int d = lane + i * kWave;
      rowv[i] = d < D ? (q4 ? kv4_elem(qrow, d, D, a.rope_dim) : load_elem(src, a.dtype, off + d)) : 0.f;
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
      rope_cos_sin(c.p, i, a.rope_dim, a.rope_log2_base, &cs, &sn);
      const float x0 = obuf[rope0 + 2 * i], x1 = obuf[rope0 + 2 * i + 1];
      obuf[rope0 + 2 * i] = x0 * cs + x1 * sn;
      obuf[rope0 + 2 * i + 1] = x1 * cs - x0 * sn;
    }
  }
  __syncthreads();
  for (int d = lane; d < D; d += kWave) store_elem(a.out, a.out_dtype, qoff + d, obuf[d]);
  __syncthreads();  // obuf is free for the next head
}

// grid (B*S, H), one wave
template <bool HCA>
__global__ __launch_bounds__(kWave) void attn_any(AttnArgs a) {
  extern __shared__ float obuf[];  // D floats
  attn_head<HCA>(a, blockIdx.x, blockIdx.y, obuf);
}

// Recompute, exactly, the queries the persistent kernel flagged (redo[qi] != 0):
// grid (ceil(B*S / 64), H), one wave; each wave checks 64 flags with one load
// and recomputes its head of the flagged ones.
template <bool HCA>
__global__ __launch_bounds__(kWave) void attn_redo(AttnArgs a, const int* redo) {
  extern __shared__ float obuf[];
  const int64_t nq = int64_t(a.B) * a.S;
  const int64_t q0 = int64_t(blockIdx.x) * kWave;
  const int64_t mine = q0 + threadIdx.x;
  uint64_t todo = __ballot(mine < nq && redo[mine] != 0);
  while (todo != 0) {
    const int l = __builtin_ctzll(todo);
    todo &= todo - 1;
    attn_head<HCA>(a, q0 + l, blockIdx.y, obuf);
  }
}

}  // namespace

AttnPlan plan_attn(int B, int S, int H, int D, int window, int nsel, int dtype, bool hca, bool paged) {
  AttnPlan p{false, false, 1, 0, 0};
  p.mfma = (dtype == CSA_BF16 || dtype == CSA_KV4) && H == kH && D == kD;
  if (!p.mfma) return p;
  const int64_t max_cand = int64_t(window) + nsel;
  const int64_t nq = int64_t(B) * S;
  int64_t want = nq > 0 ? (kTargetBlocks + nq - 1) / nq : 1;
  const int64_t most = (max_cand + kMinSplitRows - 1) / kMinSplitRows;
  if (want > most) want = most;
  if (want > kMaxSplits) want = kMaxSplits;
  if (want < 1) want = 1;
  int64_t rows = (max_cand + want - 1) / want;
  rows = (rows + kSplitGrain - 1) / kSplitGrain * kSplitGrain;
  if (rows < kSplitGrain) rows = kSplitGrain;
  if ((!hca || paged) && rows > kMaxChunk) rows = kMaxChunk;  // chunks resolved into the code table
  p.chunk_rows = int(rows);
  p.nsplit = int((max_cand + rows - 1) / rows);
  if (p.nsplit < 1) p.nsplit = 1;
  if (p.nsplit > kMaxSplits) {  // more CSA candidates than the split table holds
    p = AttnPlan{false, false, 1, 0, 0};
    return p;
  }
  if (p.nsplit > 1) {
    p.ws_bytes = size_t(nq) * p.nsplit * (size_t(kPartialVecs) * 16 + kH * 4 * sizeof(float));
  } else if (nq >= kPersistMinQueries && (hca || nsel <= kPMaxSel) && dtype != CSA_KV4 && !paged) {
    // (quantised and paged caches take one workgroup per query instead)
    p.persist = true;
    p.ws_bytes = size_t(nq) * sizeof(int);  // per-query recompute flags
  }
  return p;
}

hipError_t launch_attn(const AttnArgs& a, const AttnPlan& plan, bool hca, hipStream_t stream) {
  const int64_t nq = int64_t(a.B) * a.S;
  if (nq == 0) return hipSuccess;
  if (plan.persist) {
    int64_t G = (nq + kPMaxQ - 1) / kPMaxQ;
    if (G < kTargetBlocks) G = kTargetBlocks;
    if (G > nq) G = nq;
    int* redo = static_cast<int*>(a.ws);
    const dim3 redo_grid(unsigned((nq + kWave - 1) / kWave), a.H);
    if (hca) {
      hipLaunchKernelGGL((attn_persist<true>), dim3(unsigned(G)), dim3(kThreads), 0, stream, a, redo);
      hipLaunchKernelGGL((attn_redo<true>), redo_grid, dim3(kWave), a.D * sizeof(float), stream, a, redo);
    } else {
      hipLaunchKernelGGL((attn_persist<false>), dim3(unsigned(G)), dim3(kThreads), 0, stream, a, redo);
      hipLaunchKernelGGL((attn_redo<false>), redo_grid, dim3(kWave), a.D * sizeof(float), stream, a, redo);
    }
  } else if (plan.mfma) {
    const dim3 grid(unsigned(nq), plan.nsplit);
    const bool split = plan.nsplit > 1;
#define CSA_ATTN_MFMA(H_, S_, Q_) \
  hipLaunchKernelGGL((attn_mfma<H_, S_, Q_>), grid, dim3(kThreads), 0, stream, a, plan.nsplit, plan.chunk_rows)
    if (a.cmp_q4) {
      if (hca && split) CSA_ATTN_MFMA(true, true, true);
      else if (hca) CSA_ATTN_MFMA(true, false, true);
      else if (split) CSA_ATTN_MFMA(false, true, true);
      else CSA_ATTN_MFMA(false, false, true);
    } else {
      if (hca && split) CSA_ATTN_MFMA(true, true, false);
      else if (hca) CSA_ATTN_MFMA(true, false, false);
      else if (split) CSA_ATTN_MFMA(false, true, false);
      else CSA_ATTN_MFMA(false, false, false);
    }
#undef CSA_ATTN_MFMA
    if (plan.nsplit > 1) {
      const dim3 grid(unsigned(nq), kPartialVecs / kWave);
      const size_t rec = size_t(3) * plan.nsplit * 16 * sizeof(float);
      if (plan.nsplit <= 16) hipLaunchKernelGGL((attn_combine<4>), grid, dim3(256), rec, stream, a, plan.nsplit);
      else hipLaunchKernelGGL((attn_combine<kMaxSplits / 16>), grid, dim3(256), rec, stream, a, plan.nsplit);
    }
  } else {
    const dim3 grid(unsigned(nq), a.H);
    if (hca) hipLaunchKernelGGL((attn_any<true>), grid, dim3(kWave), a.D * sizeof(float), stream, a);
    else hipLaunchKernelGGL((attn_any<false>), grid, dim3(kWave), a.D * sizeof(float), stream, a);
  }
  return hipGetLastError();
}

}  // namespace csa
