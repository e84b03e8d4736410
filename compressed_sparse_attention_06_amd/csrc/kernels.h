// Internal launch interface between the C ABI (api.cpp) and the kernels.
// Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa {

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
};
hipError_t launch_index_score(const IndexArgs& a, hipStream_t stream);

// Top-k: workspace plan shared by the size query and the launch.
struct TopkPlan {
  int levels;          // number of chunked reduction levels before the final pass
  int64_t cand_elems;  // (key, index) pairs per ping-pong buffer
  size_t ws_bytes;
};
TopkPlan plan_topk(int R, int N, int k);
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
};
struct AttnPlan {
  bool mfma;
  bool persist;  // one persistent workgroup per CU streams many queries
  int nsplit;
  int chunk_rows;
  size_t ws_bytes;
};
AttnPlan plan_attn(int B, int S, int H, int D, int window, int nsel, int dtype, bool hca);
hipError_t launch_attn(const AttnArgs& a, const AttnPlan& plan, bool hca, hipStream_t stream);

}  // namespace csa
