// Internal launch interface between the C ABI (api.cpp) and the kernels.
// Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa {

// A paged cache: entry e of sequence b lives in pool row
// (pages[b*max_pages + (e >> page_shift)] << page_shift) + (e & (page_rows-1));
// pages == nullptr means the contiguous layout.
struct PageTable {
  const int* pages;
  int max_pages;
  int page_shift;
  int pool_pages;  // pages in the pool: table entries outside [0, pool_pages) are skipped
};
// Pool row of entry e of sequence b (-1 when its page is not allocated or
// not a page of the pool).
__device__ __forceinline__ int64_t paged_row(const PageTable& pt, int b, int64_t e) {
  const int pg = pt.pages[int64_t(b) * pt.max_pages + (e >> pt.page_shift)];
  return (pg < 0 || pg >= pt.pool_pages) ? -1 : (int64_t(pg) << pt.page_shift) + (e & ((int64_t(1) << pt.page_shift) - 1));
}

struct CompressArgs {
  const void* kv;
  const void* gate;
  const void* kv_prev;
  const void* gate_prev;
  int in_dtype;
  const float* gamma;
  int B, T;
  int64_t in_bstride;
  int D, ratio, overlap, rope_dim;
  float rope_base, eps;
  double rope_log2_base;  // log2(rope_base), formed on the host
  int tok0, e0, n_entries;
  const int* pos;  // ring mode when non-null
  void* out;
  int out_dtype;
  int64_t out_bstride;
  int out_cap;
  void* ws;  // split partials and counters (zero counters on entry, left zero)
  PageTable pt;  // paged output (out is then the pool)
};
// Compressor plan, shared by the workspace-size query and the launch.
struct CompressPlan {
  bool lanes;       // D a multiple of 128: the lane kernel (else one wave per entry)
  int cpl;          // channels per lane (2, 4 or 8)
  int gc, gr;       // waves per block: channel groups x candidate groups
  int nsplit;       // blocks per entry (long candidate lists of few entries)
  size_t ws_bytes;  // split partial states + one arrival counter per entry
};
CompressPlan plan_compress(int64_t entries, int D, int ratio, int overlap);
// Launch independent compressor jobs; jobs that share a lane layout run in
// one kernel (results identical to one launch per job).
hipError_t launch_compress(const CompressArgs* jobs, const CompressPlan* plans, int n, hipStream_t stream);

struct IndexArgs {
  const void* q_idx;
  const float* w;
  const void* cache;
  int dtype;
  const int* pos;
  int B, S, H, D, Ncap, ratio;
  float* scores;
  bool use_mfma;  // bf16, 64 heads x 128, 16-byte aligned operands
  PageTable pt;   // paged index cache (cache is then the pool)
};
hipError_t launch_index_score(const IndexArgs& a, hipStream_t stream);

// Top-k: workspace plan shared by the size query and the launch.
struct TopkPlan {
  int levels;          // number of chunked reduction levels before the final pass
  int64_t cand_elems;  // (key, index) pairs per ping-pong buffer
  size_t ws_bytes;
};
TopkPlan plan_topk(int R, int N, int k);
// Device address of the current device's top-k scratch array
// (CSA_TOPK_NOALLOC_SCRATCH_BYTES), looked up on first use per device.
hipError_t topk_scratch(void** out);
hipError_t launch_topk(const float* scores, const int* n_valid, int R, int N, int k, int* idx,
                       void* ws, hipStream_t stream);

struct AttnArgs {
  const void* q;
  const void* cmp;
  int Ncap;
  const int* idx;  // CSA selection, or null for HCA
  int k;
  int ratio;       // HCA visibility ratio
  const void* win;
  int Wcap, window;
  const int* pos;
  const float* sink;
  int dtype;
  float scale;
  int rope_dim;
  float rope_base;
  double rope_log2_base;  // log2(rope_base), formed on the host
  int B, S, H, D;
  void* out;
  int out_dtype;
  void* ws;
  int cmp_q4;         // cmp rows are quantised (kv4.h); q and win are then bf16
  int cmp_row_bytes;  // bytes per quantised cmp row
  PageTable pt;       // paged compressed cache (cmp is then the pool)
};
struct AttnPlan {
  bool mfma;
  bool persist;  // one persistent workgroup per CU streams many queries
  int nsplit;
  int chunk_rows;
  size_t ws_bytes;
};
AttnPlan plan_attn(int B, int S, int H, int D, int window, int nsel, int dtype, bool hca, bool paged = false);
hipError_t launch_attn(const AttnArgs& a, const AttnPlan& plan, bool hca, hipStream_t stream);

// Quantisation of rows into the FP4/FP8 cache format of kv4.h.
struct Kv4Args {
  const void* x;
  int x_dtype;
  int64_t rows;
  int D, rope_dim, row_bytes;
  void* out;
};
hipError_t launch_kv4_quantize(const Kv4Args& a, hipStream_t stream);

// Projection GEMM C[g][m][n] = sum_k A[g][m][k] * W[g][n][k] (bf16 weights,
// bf16 or fp32 activations, fp32 accumulation), g < groups.  Requires
// K % 128 == 0 and N % 16 == 0; pointers 16-byte aligned.
struct ProjArgs {
  const void* A;
  int a_dtype;      // CSA_BF16 or CSA_F32 (split into two bf16 products)
  int64_t lda;      // elements between token rows of A
  int64_t a_goff;   // elements between groups of A (along a row)
  const void* W;    // bf16 [groups][N][K]
  int64_t w_goff;   // elements between groups of W
  void* C;
  int c_dtype;
  int64_t ldc;
  int64_t c_goff;
  int M, N, K, groups;
  int a_nsum;            // fp32 A: sum of a_nsum partial arrays a_kstride apart
  int64_t a_kstride;
  int kc, ks_count;      // K chunk and chunk count (plan_proj)
  float* part;           // ks_count > 1: fp32 partials [ks][..C layout..]
  int64_t part_kstride;
};
// K chunking of one projection product: token tiles per block (mt), K chunk
// (kc), chunks (ks) and token chunks.
struct ProjPlan {
  int mt, kc, ks, mchunks;
};
ProjPlan plan_proj(int M, int N, int K, int groups, bool act_f32);
hipError_t launch_proj_gemm(const ProjArgs& a, hipStream_t stream);
// C = sum of the ks_count partials of a (in chunk order).
hipError_t launch_proj_reduce(const ProjArgs& a, hipStream_t stream);

// Row normalisation y = x / sqrt(mean(x^2) + eps) * gamma over column groups
// of G, then RoPE of each group's trailing rope_dim at pos[m].
struct NormArgs {
  const float* x;
  int64_t ldx;
  int x_nsum;          // x is the sum of x_nsum partial arrays x_kstride apart
  int64_t x_kstride;
  const float* gamma;  // [G] or null (no gain)
  const int* pos;      // [M] or null (with rope_dim == 0)
  void* y;
  int y_dtype;
  int64_t ldy;
  int M, G, rope_dim;
  double rope_log2_base;
  float eps;
};
hipError_t launch_rows_norm(const NormArgs& a, int ngroups, hipStream_t stream);

}  // namespace csa
