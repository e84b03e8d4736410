// C ABI entry points: argument validation (host only, before any HIP call)
// and dispatch to the gfx950 kernels.  See include/csa.h for the contract.
#include <cmath>
#include <cstdint>

#include "csa.h"
#include "kernels.h"

namespace {

constexpr int kVersion = 10000;  // 1.0.0
constexpr int64_t kMaxGridY = 65535;

bool dtype_ok(int d) { return d == CSA_F32 || d == CSA_BF16; }
int esize(int d) { return d == CSA_BF16 ? 2 : 4; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int hip_status(hipError_t e) { return e == hipSuccess ? CSA_OK : CSA_ERR_HIP; }

}  // namespace

extern "C" {

const char* csa_status_string(int status) {
  switch (status) {
    case CSA_OK: return "ok";
    case CSA_ERR_INVALID_ARG: return "invalid argument";
    case CSA_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case CSA_ERR_HIP: return "HIP runtime error";
    case CSA_ERR_WORKSPACE: return "workspace too small";
    default: return "unknown status";
  }
}

int csa_version(void) { return kVersion; }

size_t csa_compress_workspace_size(int64_t entries, int D, int ratio, int overlap) {
  if (entries < 0 || D < 1 || D > 8192 || ratio < 1 || (overlap != 0 && overlap != 1)) return 0;
  return csa::plan_compress(entries, D, ratio, overlap).ws_bytes;
}

}  // extern "C"

namespace {

// Validates one compressor call and fills its kernel arguments and plan.
int compress_job(const csa_compress_job& j, csa::CompressArgs* out_args, csa::CompressPlan* out_plan) {
  if (!j.kv || !j.gate || !j.gamma || !j.out) return CSA_ERR_INVALID_ARG;
  if (!dtype_ok(j.in_dtype) || !dtype_ok(j.out_dtype)) return CSA_ERR_INVALID_ARG;
  if (j.B < 0 || j.T < 1 || j.D < 1 || j.ratio < 1 || (j.overlap != 0 && j.overlap != 1)) return CSA_ERR_INVALID_ARG;
  if (j.rope_dim < 0 || j.rope_dim % 2 != 0 || j.rope_dim > j.D) return CSA_ERR_INVALID_ARG;
  if (!(j.eps >= 0.f) || !std::isfinite(j.eps) || !(j.rope_base > 0.f) || !std::isfinite(j.rope_base))
    return CSA_ERR_INVALID_ARG;
  if (j.out_cap < 0 || j.in_bstride < int64_t(j.T) * j.D || j.out_bstride < int64_t(j.out_cap) * j.D)
    return CSA_ERR_INVALID_ARG;
  if (j.D > 8192) return CSA_ERR_UNSUPPORTED;
  if (j.pos == nullptr) {
    if (j.tok0 < 0 || j.e0 < 0 || j.n_entries < 0 || int64_t(j.e0) + j.n_entries > j.out_cap)
      return CSA_ERR_INVALID_ARG;
    if (j.n_entries > 0) {
      const int64_t lo = (int64_t(j.e0) - ((j.overlap && j.e0 > 0) ? 1 : 0)) * j.ratio;
      const int64_t hi = (int64_t(j.e0) + j.n_entries) * j.ratio;
      if (lo < j.tok0 || hi > int64_t(j.tok0) + j.T) return CSA_ERR_INVALID_ARG;
    }
  } else {
    if (int64_t(j.T) < int64_t(1 + j.overlap) * j.ratio) return CSA_ERR_INVALID_ARG;
  }
  const int64_t entries = j.pos == nullptr ? int64_t(j.B) * j.n_entries : j.B;
  if (entries > INT32_MAX) return CSA_ERR_UNSUPPORTED;
  const csa::CompressPlan plan = csa::plan_compress(entries, j.D, j.ratio, j.overlap);
  if (plan.ws_bytes > 0 && (j.ws == nullptr || j.ws_bytes < plan.ws_bytes)) return CSA_ERR_WORKSPACE;
  if (plan.ws_bytes > 0 && !aligned16(j.ws)) return CSA_ERR_INVALID_ARG;
  csa::CompressArgs a{};
  a.kv = j.kv;
  a.gate = j.gate;
  a.kv_prev = j.kv_prev ? j.kv_prev : j.kv;
  a.gate_prev = j.gate_prev ? j.gate_prev : j.gate;
  a.in_dtype = j.in_dtype;
  a.gamma = j.gamma;
  a.B = j.B;
  a.T = j.T;
  a.in_bstride = j.in_bstride;
  a.D = j.D;
  a.ratio = j.ratio;
  a.overlap = j.overlap;
  a.rope_dim = j.rope_dim;
  a.rope_base = j.rope_base;
  a.rope_log2_base = std::log2(double(j.rope_base));
  a.eps = j.eps;
  a.tok0 = j.tok0;
  a.e0 = j.e0;
  a.n_entries = j.n_entries;
  a.pos = j.pos;
  a.out = j.out;
  a.out_dtype = j.out_dtype;
  a.out_bstride = j.out_bstride;
  a.out_cap = j.out_cap;
  a.ws = j.ws;
  *out_args = a;
  *out_plan = plan;
  return CSA_OK;
}

}  // namespace

extern "C" {

int csa_compress(const void* kv, const void* gate, const void* kv_prev, const void* gate_prev, int in_dtype,
                 const float* gamma, int B, int T, int64_t in_bstride, int D, int ratio, int overlap,
                 int rope_dim, float rope_base, float eps, int tok0, int e0, int n_entries, const int* pos,
                 void* out, int out_dtype, int64_t out_bstride, int out_cap, void* ws, size_t ws_bytes,
                 hipStream_t stream) {
  const csa_compress_job j{kv,   gate,  kv_prev, gate_prev, in_dtype, gamma,     B,         T,       in_bstride,
                           D,    ratio, overlap, rope_dim,  rope_base, eps,      tok0,      e0,      n_entries,
                           pos,  out,   out_dtype, out_bstride, out_cap, ws,      ws_bytes};
  csa::CompressArgs a;
  csa::CompressPlan plan;
  const int st = compress_job(j, &a, &plan);
  if (st != CSA_OK) return st;
  return hip_status(csa::launch_compress(&a, &plan, 1, stream));
}

int csa_compress_jobs(const csa_compress_job* jobs, int n_jobs, hipStream_t stream) {
  if (n_jobs < 0 || n_jobs > CSA_MAX_COMPRESS_JOBS || (n_jobs > 0 && jobs == nullptr)) return CSA_ERR_INVALID_ARG;
  csa::CompressArgs a[CSA_MAX_COMPRESS_JOBS];
  csa::CompressPlan plan[CSA_MAX_COMPRESS_JOBS];
  for (int i = 0; i < n_jobs; ++i) {
    const int st = compress_job(jobs[i], &a[i], &plan[i]);
    if (st != CSA_OK) return st;
  }
  return hip_status(csa::launch_compress(a, plan, n_jobs, stream));
}

int csa_index_score(const void* q_idx, const float* w, const void* idx_cache, int dtype, const int* pos, int B,
                    int S, int H_I, int D_I, int Ncap, int ratio, float* scores, hipStream_t stream) {
  if (!q_idx || !w || !idx_cache || !pos || !scores) return CSA_ERR_INVALID_ARG;
  if (!dtype_ok(dtype) || B < 0 || S < 0 || H_I < 1 || D_I < 1 || Ncap < 0 || ratio < 1) return CSA_ERR_INVALID_ARG;
  if (int64_t(B) * S > INT32_MAX || (int64_t(Ncap) + 255) / 256 > kMaxGridY) return CSA_ERR_UNSUPPORTED;
  const bool mfma = dtype == CSA_BF16 && H_I == 64 && D_I == 128 && aligned16(q_idx) && aligned16(idx_cache) &&
                    aligned16(scores);  // the matrix-core kernels store scores in 16-byte groups
  if (!mfma && int64_t(H_I) * D_I + H_I > 16384) return CSA_ERR_UNSUPPORTED;
  csa::IndexArgs a{};
  a.q_idx = q_idx;
  a.w = w;
  a.cache = idx_cache;
  a.dtype = dtype;
  a.use_mfma = mfma;
  a.pos = pos;
  a.B = B;
  a.S = S;
  a.H = H_I;
  a.D = D_I;
  a.Ncap = Ncap;
  a.ratio = ratio;
  a.scores = scores;
  return hip_status(csa::launch_index_score(a, stream));
}

size_t csa_topk_workspace_size(int R, int N, int k) {
  if (R < 0 || N < 0 || k < 1 || k > 4096) return 0;
  return csa::plan_topk(R, N, k).ws_bytes;
}

int csa_topk(const float* scores, const int* n_valid, int R, int N, int k, int* idx, void* ws, size_t ws_bytes,
             hipStream_t stream) {
  if (!scores || !idx || R < 0 || N < 0 || k < 1 || k > 4096) return CSA_ERR_INVALID_ARG;
  if (R > INT32_MAX / 2) return CSA_ERR_UNSUPPORTED;
  const csa::TopkPlan plan = csa::plan_topk(R, N, k);
  if (plan.ws_bytes > 0 && (ws == nullptr || ws_bytes < plan.ws_bytes)) return CSA_ERR_WORKSPACE;
  if ((int64_t(N) + 16383) / 16384 > kMaxGridY) return CSA_ERR_UNSUPPORTED;
  return hip_status(csa::launch_topk(scores, n_valid, R, N, k, idx, ws, stream));
}

namespace {

int attn_common(const void* q, const void* cmp, int Ncap, const int* idx, int k, int ratio, const void* win, int Wcap,
                int window, const int* pos, const float* sink, int dtype, float scale, int rope_dim, float rope_base,
                int B, int S, int H, int D, void* out, int out_dtype, void* ws, size_t ws_bytes, bool hca,
                hipStream_t stream) {
  if (!q || !cmp || !pos || !sink || !out || (!hca && !idx) || (window > 0 && !win)) return CSA_ERR_INVALID_ARG;
  if (!dtype_ok(dtype) || !dtype_ok(out_dtype)) return CSA_ERR_INVALID_ARG;
  if (B < 0 || S < 0 || H < 1 || D < 2 || Ncap < 0 || window < 0 || Wcap < window || (!hca && k < 0) ||
      (hca && ratio < 1))
    return CSA_ERR_INVALID_ARG;
  if (window > 0 && Wcap < 1) return CSA_ERR_INVALID_ARG;
  if (rope_dim < 0 || rope_dim % 2 != 0 || rope_dim > D) return CSA_ERR_INVALID_ARG;
  if (!std::isfinite(scale) || !(rope_base > 0.f) || !std::isfinite(rope_base)) return CSA_ERR_INVALID_ARG;
  if (int64_t(B) * S > INT32_MAX) return CSA_ERR_UNSUPPORTED;
  const int64_t max_cand = int64_t(window) + (hca ? Ncap : k);
  if (max_cand > INT32_MAX) return CSA_ERR_UNSUPPORTED;
  csa::AttnPlan plan = csa::plan_attn(B, S, H, D, window, hca ? Ncap : k, dtype, hca);
  if (plan.mfma && !(aligned16(q) && aligned16(cmp) && (window == 0 || aligned16(win)) && aligned16(out)))
    plan = csa::AttnPlan{false, false, 1, 0, 0};
  if (!plan.mfma && D > 1024) return CSA_ERR_UNSUPPORTED;
  if (plan.nsplit > kMaxGridY) return CSA_ERR_UNSUPPORTED;
  if (plan.ws_bytes > 0 && (ws == nullptr || ws_bytes < plan.ws_bytes)) return CSA_ERR_WORKSPACE;
  if (plan.ws_bytes > 0 && !aligned16(ws)) return CSA_ERR_INVALID_ARG;
  csa::AttnArgs a{};
  a.q = q;
  a.cmp = cmp;
  a.Ncap = Ncap;
  a.idx = idx;
  a.k = k;
  a.ratio = ratio;
  a.win = win;
  a.Wcap = Wcap;
  a.window = window;
  a.pos = pos;
  a.sink = sink;
  a.dtype = dtype;
  a.scale = scale;
  a.rope_dim = rope_dim;
  a.rope_base = rope_base;
  a.rope_log2_base = std::log2(double(rope_base));
  a.B = B;
  a.S = S;
  a.H = H;
  a.D = D;
  a.out = out;
  a.out_dtype = out_dtype;
  a.ws = ws;
  return hip_status(csa::launch_attn(a, plan, hca, stream));
}

size_t attn_ws(int B, int S, int H, int D, int window, int nsel, bool hca) {
  if (B < 0 || S < 0 || H < 1 || D < 2 || window < 0 || nsel < 0 || int64_t(window) + nsel > INT32_MAX) return 0;
  return csa::plan_attn(B, S, H, D, window, nsel, CSA_BF16, hca).ws_bytes;
}

}  // namespace

size_t csa_sparse_attn_workspace_size(int B, int S, int H, int D, int k, int window) {
  if (k < 0 || window < 0) return 0;
  return attn_ws(B, S, H, D, window, k, false);
}

int csa_sparse_attn(const void* q, const void* cmp, int Ncap, const int* idx, int k, const void* win, int Wcap,
                    int window, const int* pos, const float* sink, int dtype, float scale, int rope_dim,
                    float rope_base, int B, int S, int H, int D, void* out, int out_dtype, void* ws, size_t ws_bytes,
                    hipStream_t stream) {
  return attn_common(q, cmp, Ncap, idx, k, 1, win, Wcap, window, pos, sink, dtype, scale, rope_dim, rope_base, B, S,
                     H, D, out, out_dtype, ws, ws_bytes, false, stream);
}

size_t hca_attn_workspace_size(int B, int S, int H, int D, int Ncap, int window) {
  if (Ncap < 0 || window < 0) return 0;
  return attn_ws(B, S, H, D, window, Ncap, true);
}

int hca_attn(const void* q, const void* cmp, int Ncap, int ratio, const void* win, int Wcap, int window,
             const int* pos, const float* sink, int dtype, float scale, int rope_dim, float rope_base, int B, int S,
             int H, int D, void* out, int out_dtype, void* ws, size_t ws_bytes, hipStream_t stream) {
  return attn_common(q, cmp, Ncap, nullptr, 0, ratio, win, Wcap, window, pos, sink, dtype, scale, rope_dim,
                     rope_base, B, S, H, D, out, out_dtype, ws, ws_bytes, true, stream);
}

}  // extern "C"
