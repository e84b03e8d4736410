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

int csa_compress(const void* kv, const void* gate, const void* kv_prev, const void* gate_prev, int in_dtype,
                 const float* gamma, int B, int T, int64_t in_bstride, int D, int ratio, int overlap,
                 int rope_dim, float rope_base, float eps, int tok0, int e0, int n_entries, const int* pos,
                 void* out, int out_dtype, int64_t out_bstride, int out_cap, void* ws, size_t ws_bytes,
                 hipStream_t stream) {
  if (!kv || !gate || !gamma || !out) return CSA_ERR_INVALID_ARG;
  if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype)) return CSA_ERR_INVALID_ARG;
  if (B < 0 || T < 1 || D < 1 || ratio < 1 || (overlap != 0 && overlap != 1)) return CSA_ERR_INVALID_ARG;
  if (rope_dim < 0 || rope_dim % 2 != 0 || rope_dim > D) return CSA_ERR_INVALID_ARG;
  if (!(eps >= 0.f) || !std::isfinite(eps) || !(rope_base > 0.f) || !std::isfinite(rope_base))
    return CSA_ERR_INVALID_ARG;
  if (out_cap < 0 || in_bstride < int64_t(T) * D || out_bstride < int64_t(out_cap) * D) return CSA_ERR_INVALID_ARG;
  if (D > 8192) return CSA_ERR_UNSUPPORTED;
  if (pos == nullptr) {
    if (tok0 < 0 || e0 < 0 || n_entries < 0 || int64_t(e0) + n_entries > out_cap) return CSA_ERR_INVALID_ARG;
    if (n_entries > 0) {
      const int64_t lo = (int64_t(e0) - ((overlap && e0 > 0) ? 1 : 0)) * ratio;
      const int64_t hi = (int64_t(e0) + n_entries) * ratio;
      if (lo < tok0 || hi > int64_t(tok0) + T) return CSA_ERR_INVALID_ARG;
    }
  } else {
    if (int64_t(T) < int64_t(1 + overlap) * ratio) return CSA_ERR_INVALID_ARG;
  }
  const int64_t entries = pos == nullptr ? int64_t(B) * n_entries : B;
  if (entries > INT32_MAX) return CSA_ERR_UNSUPPORTED;
  const csa::CompressPlan plan = csa::plan_compress(entries, D, ratio, overlap);
  if (plan.ws_bytes > 0 && (ws == nullptr || ws_bytes < plan.ws_bytes)) return CSA_ERR_WORKSPACE;
  if (plan.ws_bytes > 0 && !aligned16(ws)) return CSA_ERR_INVALID_ARG;
  csa::CompressArgs a{};
  a.kv = kv;
  a.gate = gate;
  a.kv_prev = kv_prev ? kv_prev : kv;
  a.gate_prev = gate_prev ? gate_prev : gate;
  a.in_dtype = in_dtype;
  a.gamma = gamma;
  a.B = B;
  a.T = T;
  a.in_bstride = in_bstride;
  a.D = D;
  a.ratio = ratio;
  a.overlap = overlap;
  a.rope_dim = rope_dim;
  a.rope_base = rope_base;
  a.rope_log2_base = std::log2(double(rope_base));
  a.eps = eps;
  a.tok0 = tok0;
  a.e0 = e0;
  a.n_entries = n_entries;
  a.pos = pos;
  a.out = out;
  a.out_dtype = out_dtype;
  a.out_bstride = out_bstride;
  a.out_cap = out_cap;
  a.ws = ws;
  return hip_status(csa::launch_compress(a, plan, stream));
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
