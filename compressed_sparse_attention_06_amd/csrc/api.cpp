// C ABI entry points: argument validation (host only, before any HIP call)
// and dispatch to the gfx950 kernels.  See include/csa.h for the contract.
#include <cmath>
#include <cstdint>
#include <mutex>
#include <new>
#include <vector>

#include "csa.h"
#include "kernels.h"
#include "kv4.h"

namespace {

constexpr int kVersion = 10000;  // 1.0.0
constexpr int64_t kMaxGridY = 65535;

bool dtype_ok(int d) { return d == CSA_F32 || d == CSA_BF16; }
int esize(int d) { return d == CSA_BF16 ? 2 : (d == CSA_KV4 ? 1 : 4); }
// the quantised row format needs a latent and a tail in whole 32-channel blocks
bool kv4_shape_ok(int D, int rope_dim) { return D % 32 == 0 && rope_dim % 32 == 0 && rope_dim <= D; }
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
    case CSA_ERR_NO_PAGES: return "out of pages";
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

// A caller's page table, validated: page_rows a power of two >= 64, the
// logical capacity max_pages*page_rows within int32.
int page_table(const csa_page_table* t, csa::PageTable* out) {
  if (t == nullptr || t->pages == nullptr || t->max_pages < 1 || t->pool_pages < 1) return CSA_ERR_INVALID_ARG;
  if (t->page_rows < 64 || t->page_rows > (1 << 20) || (t->page_rows & (t->page_rows - 1)) != 0)
    return CSA_ERR_INVALID_ARG;
  if (int64_t(t->max_pages) * t->page_rows > INT32_MAX || int64_t(t->pool_pages) * t->page_rows > INT32_MAX)
    return CSA_ERR_UNSUPPORTED;
  int shift = 0;
  while ((1 << shift) < t->page_rows) ++shift;
  *out = csa::PageTable{t->pages, t->max_pages, shift, t->pool_pages};
  return CSA_OK;
}

// Validates one compressor call and fills its kernel arguments and plan.
int compress_job(const csa_compress_job& j, csa::CompressArgs* out_args, csa::CompressPlan* out_plan,
                 const csa::PageTable* pt = nullptr) {
  if (!dtype_ok(j.in_dtype) || !(dtype_ok(j.out_dtype) || j.out_dtype == CSA_KV4)) return CSA_ERR_INVALID_ARG;
  if (j.out_dtype == CSA_KV4 && !kv4_shape_ok(j.D, j.rope_dim)) return CSA_ERR_INVALID_ARG;
  if (j.B < 0 || j.T < 1 || j.D < 1 || j.ratio < 1 || (j.overlap != 0 && j.overlap != 1)) return CSA_ERR_INVALID_ARG;
  if (j.rope_dim < 0 || j.rope_dim % 2 != 0 || j.rope_dim > j.D) return CSA_ERR_INVALID_ARG;
  if (!(j.eps >= 0.f) || !std::isfinite(j.eps) || !(j.rope_base > 0.f) || !std::isfinite(j.rope_base))
    return CSA_ERR_INVALID_ARG;
  // (a quantised output counts its batch stride in bytes)
  const int64_t out_row = j.out_dtype == CSA_KV4 ? csa::kv4_row_bytes(j.D, j.rope_dim) : j.D;
  // (a paged output ignores out_bstride: its rows live in the pool)
  if (j.out_cap < 0 || j.in_bstride < int64_t(j.T) * j.D || (pt == nullptr && j.out_bstride < int64_t(j.out_cap) * out_row))
    return CSA_ERR_INVALID_ARG;
  if (j.out_dtype == CSA_KV4 && (!aligned16(j.out) || (pt == nullptr && j.out_bstride % 16 != 0)))
    return CSA_ERR_INVALID_ARG;
  if (j.D > 8192) return CSA_ERR_UNSUPPORTED;
  if (j.pos == nullptr) {
    if (j.tok0 < 0 || j.e0 < 0 || j.n_entries < 0) return CSA_ERR_INVALID_ARG;
    // (with no sequence nothing is built: an empty ring-mode batch, whose pos
    // is NULL, lands here and its entry range bounds nothing)
    if (j.B > 0 && int64_t(j.e0) + j.n_entries > j.out_cap) return CSA_ERR_INVALID_ARG;
    if (j.B > 0 && j.n_entries > 0) {
      const int64_t lo = (int64_t(j.e0) - ((j.overlap && j.e0 > 0) ? 1 : 0)) * j.ratio;
      const int64_t hi = (int64_t(j.e0) + j.n_entries) * j.ratio;
      if (lo < j.tok0 || hi > int64_t(j.tok0) + j.T) return CSA_ERR_INVALID_ARG;
    }
  } else {
    if (int64_t(j.T) < int64_t(1 + j.overlap) * j.ratio) return CSA_ERR_INVALID_ARG;
  }
  const int64_t entries = j.pos == nullptr ? int64_t(j.B) * j.n_entries : j.B;
  if (entries > INT32_MAX) return CSA_ERR_UNSUPPORTED;
  // a call that builds no entry reads and writes nothing: its pointers may be NULL
  const bool none = entries == 0;
  if (!none && (!j.kv || !j.gate || !j.gamma || !j.out)) return CSA_ERR_INVALID_ARG;
  const csa::CompressPlan plan = csa::plan_compress(entries, j.D, j.ratio, j.overlap);
  // the lane kernel reads and writes rows with 16-byte accesses: a misaligned
  // tensor there is rejected rather than sent down a much slower path
  if (plan.lanes) {
    const void* kvp = j.kv_prev ? j.kv_prev : j.kv;
    const void* gp = j.gate_prev ? j.gate_prev : j.gate;
    if (!aligned16(j.kv) || !aligned16(j.gate) || !aligned16(kvp) || !aligned16(gp) || !aligned16(j.out) ||
        (j.in_bstride * esize(j.in_dtype)) % 16 != 0 || (j.out_bstride * esize(j.out_dtype)) % 16 != 0)
      return CSA_ERR_INVALID_ARG;
  }
  if (!none && plan.ws_bytes > 0 && (j.ws == nullptr || j.ws_bytes < plan.ws_bytes)) return CSA_ERR_WORKSPACE;
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
  if (pt != nullptr) {
    a.pt = *pt;
    a.out_bstride = 0;
  }
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

int csa_compress_paged(const csa_compress_job* jobs, const csa_page_table* tables, int n_jobs, hipStream_t stream) {
  if (n_jobs < 0 || n_jobs > CSA_MAX_COMPRESS_JOBS || (n_jobs > 0 && (jobs == nullptr || tables == nullptr)))
    return CSA_ERR_INVALID_ARG;
  csa::CompressArgs a[CSA_MAX_COMPRESS_JOBS];
  csa::CompressPlan plan[CSA_MAX_COMPRESS_JOBS];
  for (int i = 0; i < n_jobs; ++i) {
    csa::PageTable pt{};
    csa_compress_job j = jobs[i];
    if (j.B == 0 || (j.pos == nullptr && j.n_entries == 0)) {
      j.out_cap = INT32_MAX;  // a job that builds no entry reads no page table and bounds nothing
    } else {
      const int st = page_table(&tables[i], &pt);
      if (st != CSA_OK) return st;
      j.out_cap = tables[i].max_pages * tables[i].page_rows;  // the logical capacity of a sequence
    }
    const int st = compress_job(j, &a[i], &plan[i], &pt);
    if (st != CSA_OK) return st;
  }
  return hip_status(csa::launch_compress(a, plan, n_jobs, stream));
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

}  // extern "C"

namespace {

int index_common(const void* q_idx, const float* w, const void* idx_cache, int dtype, const int* pos, int B, int S,
                 int H_I, int D_I, int Ncap, int ratio, float* scores, const csa::PageTable* pt, hipStream_t stream) {
  if (!dtype_ok(dtype) || B < 0 || S < 0 || H_I < 1 || D_I < 1 || Ncap < 0 || ratio < 1) return CSA_ERR_INVALID_ARG;
  if (int64_t(B) * S > INT32_MAX || (int64_t(Ncap) + 255) / 256 > kMaxGridY) return CSA_ERR_UNSUPPORTED;
  // no query or no cache row: nothing is read or written, the pointers may be NULL
  const bool none = int64_t(B) * S == 0 || Ncap == 0;
  if (!none && (!q_idx || !w || !idx_cache || !pos || !scores)) return CSA_ERR_INVALID_ARG;
  // matrix-core shape: 16-byte operand loads and score stores in 16-byte
  // groups, so misaligned tensors are rejected (not run on the vector path)
  const bool mfma = dtype == CSA_BF16 && H_I == 64 && D_I == 128;
  if (mfma && !(aligned16(q_idx) && aligned16(idx_cache) && aligned16(scores))) return CSA_ERR_INVALID_ARG;
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
  if (pt != nullptr) a.pt = *pt;
  return hip_status(csa::launch_index_score(a, stream));
}

}  // namespace

extern "C" {

int csa_index_score(const void* q_idx, const float* w, const void* idx_cache, int dtype, const int* pos, int B,
                    int S, int H_I, int D_I, int Ncap, int ratio, float* scores, hipStream_t stream) {
  return index_common(q_idx, w, idx_cache, dtype, pos, B, S, H_I, D_I, Ncap, ratio, scores, nullptr, stream);
}

int csa_index_score_paged(const void* q_idx, const float* w, const void* idx_pool, int dtype, const int* pos, int B,
                          int S, int H_I, int D_I, const csa_page_table* pages, int ratio, float* scores,
                          hipStream_t stream) {
  csa::PageTable pt{};
  if (int64_t(B) * S == 0)  // no query: the page table is not read
    return index_common(q_idx, w, idx_pool, dtype, pos, B, S, H_I, D_I, 0, ratio, scores, &pt, stream);
  const int st = page_table(pages, &pt);
  if (st != CSA_OK) return st;
  return index_common(q_idx, w, idx_pool, dtype, pos, B, S, H_I, D_I, pages->max_pages * pages->page_rows, ratio,
                      scores, &pt, stream);
}

size_t csa_topk_workspace_size(int R, int N, int k) {
  if (R < 0 || N < 0 || k < 1 || k > 4096) return 0;
  return csa::plan_topk(R, N, k).ws_bytes;
}

int csa_topk(const float* scores, const int* n_valid, int R, int N, int k, int* idx, void* ws, size_t ws_bytes,
             hipStream_t stream) {
  if (R < 0 || N < 0 || k < 1 || k > 4096) return CSA_ERR_INVALID_ARG;
  // no row: nothing is read or written; rows of no position read no score
  if (R > 0 && (!idx || (N > 0 && !scores))) return CSA_ERR_INVALID_ARG;
  if (R > INT32_MAX / 2) return CSA_ERR_UNSUPPORTED;
  const csa::TopkPlan plan = csa::plan_topk(R, N, k);
  if (plan.ws_bytes > 0 && (ws == nullptr || ws_bytes < plan.ws_bytes)) return CSA_ERR_WORKSPACE;
  if ((int64_t(N) + 16383) / 16384 > kMaxGridY) return CSA_ERR_UNSUPPORTED;
  return hip_status(csa::launch_topk(scores, n_valid, R, N, k, idx, ws, stream));
}

int csa_topk_noalloc(const float* scores, const int* n_valid, int R, int N, int k, int* idx, hipStream_t stream) {
  if (R < 0 || N < 0 || k < 1 || k > 4096) return CSA_ERR_INVALID_ARG;
  // no row: nothing is read or written; rows of no position read no score
  if (R > 0 && (!idx || (N > 0 && !scores))) return CSA_ERR_INVALID_ARG;
  if (R > INT32_MAX / 2) return CSA_ERR_UNSUPPORTED;
  if ((int64_t(N) + 16383) / 16384 > kMaxGridY) return CSA_ERR_UNSUPPORTED;
  const csa::TopkPlan plan = csa::plan_topk(R, N, k);
  if (plan.ws_bytes > CSA_TOPK_NOALLOC_SCRATCH_BYTES) return CSA_ERR_WORKSPACE;
  void* ws = nullptr;
  if (plan.ws_bytes > 0 && csa::topk_scratch(&ws) != hipSuccess) return CSA_ERR_HIP;
  return hip_status(csa::launch_topk(scores, n_valid, R, N, k, idx, ws, stream));
}

namespace {

int attn_common(const void* q, const void* cmp, int Ncap, const int* idx, int k, int ratio, const void* win, int Wcap,
                int window, const int* pos, const float* sink, int dtype, float scale, int rope_dim, float rope_base,
                int B, int S, int H, int D, void* out, int out_dtype, void* ws, size_t ws_bytes, bool hca,
                hipStream_t stream, const csa::PageTable* pt = nullptr) {
  if (!(dtype_ok(dtype) || dtype == CSA_KV4) || !dtype_ok(out_dtype)) return CSA_ERR_INVALID_ARG;
  if (dtype == CSA_KV4 && (!kv4_shape_ok(D, rope_dim) || !aligned16(cmp))) return CSA_ERR_INVALID_ARG;
  if (B < 0 || S < 0 || H < 1 || D < 2 || Ncap < 0 || window < 0 || Wcap < window || (!hca && k < 0) ||
      (hca && ratio < 1))
    return CSA_ERR_INVALID_ARG;
  if (window > 0 && Wcap < 1) return CSA_ERR_INVALID_ARG;
  if (rope_dim < 0 || rope_dim % 2 != 0 || rope_dim > D) return CSA_ERR_INVALID_ARG;
  if (!std::isfinite(scale) || !(rope_base > 0.f) || !std::isfinite(rope_base)) return CSA_ERR_INVALID_ARG;
  if (int64_t(B) * S > INT32_MAX) return CSA_ERR_UNSUPPORTED;
  // no query: nothing is read or written, the pointers may be NULL
  if (int64_t(B) * S == 0) return CSA_OK;
  if (!q || !cmp || !pos || !sink || !out || (!hca && !idx) || (window > 0 && !win)) return CSA_ERR_INVALID_ARG;
  const int64_t max_cand = int64_t(window) + (hca ? Ncap : k);
  if (max_cand > INT32_MAX) return CSA_ERR_UNSUPPORTED;
  csa::AttnPlan plan = csa::plan_attn(B, S, H, D, window, hca ? Ncap : k, dtype, hca, pt != nullptr);
  // matrix-core shape: rows travel in 16-byte pieces, so misaligned tensors
  // are rejected (not run on the vector path)
  if (plan.mfma && !(aligned16(q) && aligned16(cmp) && (window == 0 || aligned16(win)) && aligned16(out)))
    return CSA_ERR_INVALID_ARG;
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
  if (dtype == CSA_KV4) {  // bf16 queries and window rows, quantised compressed rows
    a.dtype = CSA_BF16;
    a.cmp_q4 = 1;
    a.cmp_row_bytes = csa::kv4_row_bytes(D, rope_dim);
  }
  if (pt != nullptr) a.pt = *pt;
  return hip_status(csa::launch_attn(a, plan, hca, stream));
}

// enough for every plan of the shape: bf16 or quantised, contiguous or paged
size_t attn_ws(int B, int S, int H, int D, int window, int nsel, bool hca) {
  if (B < 0 || S < 0 || H < 1 || D < 2 || window < 0 || nsel < 0 || int64_t(window) + nsel > INT32_MAX) return 0;
  size_t ws = 0;
  for (int dt : {CSA_BF16, CSA_KV4})
    for (bool paged : {false, true}) {
      const size_t w = csa::plan_attn(B, S, H, D, window, nsel, dt, hca, paged).ws_bytes;
      ws = w > ws ? w : ws;
    }
  return ws;
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

int csa_sparse_attn_paged(const void* q, const void* cmp_pool, const csa_page_table* pages, const int* idx, int k,
                          const void* win, int Wcap, int window, const int* pos, const float* sink, int dtype,
                          float scale, int rope_dim, float rope_base, int B, int S, int H, int D, void* out,
                          int out_dtype, void* ws, size_t ws_bytes, hipStream_t stream) {
  csa::PageTable pt{};
  const bool none = int64_t(B) * S == 0;  // no query: the page table is not read
  const int st = none ? CSA_OK : page_table(pages, &pt);
  if (st != CSA_OK) return st;
  return attn_common(q, cmp_pool, none ? 0 : pages->max_pages * pages->page_rows, idx, k, 1, win, Wcap, window, pos, sink, dtype,
                     scale, rope_dim, rope_base, B, S, H, D, out, out_dtype, ws, ws_bytes, false, stream, &pt);
}

int hca_attn_paged(const void* q, const void* cmp_pool, const csa_page_table* pages, int ratio, const void* win,
                   int Wcap, int window, const int* pos, const float* sink, int dtype, float scale, int rope_dim,
                   float rope_base, int B, int S, int H, int D, void* out, int out_dtype, void* ws, size_t ws_bytes,
                   hipStream_t stream) {
  csa::PageTable pt{};
  const bool none = int64_t(B) * S == 0;  // no query: the page table is not read
  const int st = none ? CSA_OK : page_table(pages, &pt);
  if (st != CSA_OK) return st;
  return attn_common(q, cmp_pool, none ? 0 : pages->max_pages * pages->page_rows, nullptr, 0, ratio, win, Wcap, window, pos, sink,
                     dtype, scale, rope_dim, rope_base, B, S, H, D, out, out_dtype, ws, ws_bytes, true, stream, &pt);
}

// ---------------------------------------------------------------------------
// Page pool: which pages of a caller-owned device pool are free (host only)
// ---------------------------------------------------------------------------
struct csa_page_pool {
  std::mutex mu;
  std::vector<int> free_pages;  // a stack: the lowest-numbered free page on top after creation
  std::vector<unsigned char> used;
};

csa_page_pool* csa_page_pool_create(int n_pages) {
  if (n_pages < 1) return nullptr;
  csa_page_pool* p = new (std::nothrow) csa_page_pool;
  if (p == nullptr) return nullptr;
  try {
    p->free_pages.resize(size_t(n_pages));
    for (int i = 0; i < n_pages; ++i) p->free_pages[size_t(i)] = n_pages - 1 - i;
    p->used.assign(size_t(n_pages), 0);
  } catch (...) {
    delete p;
    return nullptr;
  }
  return p;
}

void csa_page_pool_destroy(csa_page_pool* pool) { delete pool; }

int csa_page_pool_available(csa_page_pool* pool) {
  if (pool == nullptr) return CSA_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lock(pool->mu);
  return int(pool->free_pages.size());
}

int csa_page_pool_alloc(csa_page_pool* pool, int n, int* pages) {
  if (pool == nullptr || n < 0 || (n > 0 && pages == nullptr)) return CSA_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lock(pool->mu);
  if (size_t(n) > pool->free_pages.size()) return CSA_ERR_NO_PAGES;
  for (int i = 0; i < n; ++i) {
    pages[i] = pool->free_pages.back();
    pool->free_pages.pop_back();
    pool->used[size_t(pages[i])] = 1;
  }
  return CSA_OK;
}

int csa_page_pool_release(csa_page_pool* pool, int n, const int* pages) {
  if (pool == nullptr || n < 0 || (n > 0 && pages == nullptr)) return CSA_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lock(pool->mu);
  // all or nothing: every page must be in use and named once
  std::vector<unsigned char> seen;
  for (int i = 0; i < n; ++i) {
    const int pg = pages[i];
    if (pg < 0 || size_t(pg) >= pool->used.size() || !pool->used[size_t(pg)]) return CSA_ERR_INVALID_ARG;
    if (seen.empty()) seen.assign(pool->used.size(), 0);
    if (seen[size_t(pg)]) return CSA_ERR_INVALID_ARG;
    seen[size_t(pg)] = 1;
  }
  for (int i = n - 1; i >= 0; --i) {
    pool->used[size_t(pages[i])] = 0;
    pool->free_pages.push_back(pages[i]);
  }
  return CSA_OK;
}

int csa_page_table_reserve(csa_page_pool* pool, int* row, int max_pages, int page_rows, int64_t n_entries) {
  if (pool == nullptr || row == nullptr || max_pages < 1 || page_rows < 1 || n_entries < 0) return CSA_ERR_INVALID_ARG;
  const int64_t need = (n_entries + page_rows - 1) / page_rows;
  if (need > max_pages) return CSA_ERR_INVALID_ARG;
  int missing = 0;
  for (int64_t j = 0; j < need; ++j) missing += row[j] < 0 ? 1 : 0;
  if (missing == 0) return CSA_OK;
  std::vector<int> got(size_t(missing), -1);
  const int st = csa_page_pool_alloc(pool, missing, got.data());
  if (st != CSA_OK) return st;  // nothing taken
  int k = 0;
  for (int64_t j = 0; j < need; ++j)
    if (row[j] < 0) row[j] = got[size_t(k++)];
  return CSA_OK;
}

int csa_page_table_release(csa_page_pool* pool, int* row, int max_pages) {
  if (pool == nullptr || row == nullptr || max_pages < 1) return CSA_ERR_INVALID_ARG;
  std::vector<int> held;
  for (int j = 0; j < max_pages; ++j)
    if (row[j] >= 0) held.push_back(row[j]);
  const int st = csa_page_pool_release(pool, int(held.size()), held.data());
  if (st != CSA_OK) return st;
  for (int j = 0; j < max_pages; ++j) row[j] = -1;
  return CSA_OK;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Projections on either side of the attention
// ---------------------------------------------------------------------------
namespace {

bool proj_dims_ok(int M, int N, int K) { return M >= 0 && N > 0 && K > 0 && N % 16 == 0 && K % 128 == 0; }

}  // namespace

namespace {

// fp32 workspace layout of the query path: latent partials, normalised
// latent, head partials (floats)
struct QPlan {
  csa::ProjPlan p1, p2;
  size_t part1, qrn, qf;
};
QPlan q_plan(int M, int d_model, int q_rank, int64_t hq) {
  QPlan q;
  q.p1 = csa::plan_proj(M, q_rank, d_model, 1, false);
  q.p2 = csa::plan_proj(M, int(hq), q_rank, 1, true);
  q.part1 = size_t(q.p1.ks) * M * q_rank;
  q.qrn = size_t(M) * q_rank;
  q.qf = size_t(q.p2.ks) * M * hq;
  return q;
}

struct OPlan {
  csa::ProjPlan pa, pb;
  size_t r, y;
};
OPlan o_plan(int M, int groups, int o_rank, int64_t kg, int d_model, bool o_f32) {
  OPlan o;
  o.pa = csa::plan_proj(M, o_rank, int(kg), groups, o_f32);
  o.pb = csa::plan_proj(M, d_model, groups * o_rank, 1, true);
  o.r = size_t(o.pa.ks) * M * groups * o_rank;
  o.y = o.pb.ks > 1 ? size_t(o.pb.ks) * M * d_model : 0;
  return o;
}

}  // namespace

extern "C" {

size_t csa_kv4_row_bytes(int D, int rope_dim) {
  if (D < 1 || rope_dim < 0 || !kv4_shape_ok(D, rope_dim)) return 0;
  return size_t(csa::kv4_row_bytes(D, rope_dim));
}

int csa_kv4_quantize(const void* x, int x_dtype, int64_t rows, int D, int rope_dim, void* out, hipStream_t stream) {
  if (!dtype_ok(x_dtype) || rows < 0 || D < 1 || rope_dim < 0 || !kv4_shape_ok(D, rope_dim))
    return CSA_ERR_INVALID_ARG;
  if (rows > 0 && (!x || !out)) return CSA_ERR_INVALID_ARG;  // no row: the pointers may be NULL
  if (D > 8192 || (rows + 3) / 4 > INT32_MAX) return CSA_ERR_UNSUPPORTED;
  if (!aligned16(out)) return CSA_ERR_INVALID_ARG;
  const csa::Kv4Args a{x, x_dtype, rows, D, rope_dim, csa::kv4_row_bytes(D, rope_dim), out};
  return hip_status(csa::launch_kv4_quantize(a, stream));
}

size_t csa_q_proj_workspace_size(int M, int d_model, int q_rank, int H, int head_dim) {
  if (M < 0 || d_model < 1 || q_rank < 1 || H < 1 || head_dim < 1) return 0;
  if (d_model % 128 != 0 || q_rank % 128 != 0 || (int64_t(H) * head_dim) % 16 != 0) return 0;
  const QPlan q = q_plan(M, d_model, q_rank, int64_t(H) * head_dim);
  return (q.part1 + q.qrn + q.qf) * sizeof(float);
}

int csa_q_proj(const void* x, const void* wq_a, const float* gamma_q, const void* wq_b, const int* pos, int M,
               int d_model, int q_rank, int H, int head_dim, int rope_dim, float rope_base, float eps, void* q,
               void* ws, size_t ws_bytes, hipStream_t stream) {
  if (M < 0 || d_model < 1 || q_rank < 1 || H < 1 || head_dim < 2) return CSA_ERR_INVALID_ARG;
  if (rope_dim < 0 || rope_dim % 2 != 0 || rope_dim > head_dim) return CSA_ERR_INVALID_ARG;
  if (!(eps >= 0.f) || !std::isfinite(eps) || !(rope_base > 0.f) || !std::isfinite(rope_base))
    return CSA_ERR_INVALID_ARG;
  const int64_t hq = int64_t(H) * head_dim;
  if (hq > INT32_MAX / 2 || int64_t(M) * hq > (int64_t(1) << 40)) return CSA_ERR_UNSUPPORTED;
  if (!proj_dims_ok(M, q_rank, d_model) || !proj_dims_ok(M, int(hq), q_rank) || q_rank > 16384 ||
      head_dim > 16384)
    return CSA_ERR_UNSUPPORTED;
  if (int64_t(M) > 65535 * 32) return CSA_ERR_UNSUPPORTED;
  if (M == 0) return CSA_OK;  // no token: nothing is read or written, the pointers may be NULL
  if (!x || !wq_a || !gamma_q || !wq_b || !q || (rope_dim > 0 && !pos)) return CSA_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(wq_a) || !aligned16(wq_b) || !aligned16(q)) return CSA_ERR_INVALID_ARG;
  const size_t need = csa_q_proj_workspace_size(M, d_model, q_rank, H, head_dim);
  if (need > 0 && (ws == nullptr || ws_bytes < need)) return CSA_ERR_WORKSPACE;
  if (need > 0 && !aligned16(ws)) return CSA_ERR_INVALID_ARG;
  const QPlan pl = q_plan(M, d_model, q_rank, hq);
  float* part1 = static_cast<float*>(ws);
  float* qrn = part1 + pl.part1;
  float* qf = qrn + pl.qrn;
  const double l2b = std::log2(double(rope_base));
  // down-projection to the latent (K-chunk partials)
  csa::ProjArgs g1{x,  CSA_BF16, d_model, 0, wq_a, 0, part1, CSA_F32, q_rank, 0, M, q_rank, d_model, 1, 1, 0,
                   pl.p1.kc, pl.p1.ks, part1, int64_t(M) * q_rank};
  if (csa::launch_proj_gemm(g1, stream) != hipSuccess) return CSA_ERR_HIP;
  // RMSNorm of the latent (summing the partials), with its gain
  csa::NormArgs n1{part1, q_rank, pl.p1.ks, int64_t(M) * q_rank, gamma_q, nullptr, qrn, CSA_F32, q_rank,
                   M,     q_rank, 0,        l2b,                 eps};
  if (csa::launch_rows_norm(n1, 1, stream) != hipSuccess) return CSA_ERR_HIP;
  // up-projection to the heads
  csa::ProjArgs g2{qrn, CSA_F32, q_rank, 0, wq_b, 0, qf, CSA_F32, hq, 0, M, int(hq), q_rank, 1, 1, 0,
                   pl.p2.kc, pl.p2.ks, qf, int64_t(M) * hq};
  if (csa::launch_proj_gemm(g2, stream) != hipSuccess) return CSA_ERR_HIP;
  // per-head RMS (no gain), RoPE on each head's trailing dims, bf16 queries
  csa::NormArgs n2{qf, hq, pl.p2.ks, int64_t(M) * hq, nullptr, pos, q, CSA_BF16, hq, M, head_dim, rope_dim, l2b,
                   eps};
  if (csa::launch_rows_norm(n2, H, stream) != hipSuccess) return CSA_ERR_HIP;
  return CSA_OK;
}

size_t csa_out_proj_workspace_size(int M, int H, int head_dim, int groups, int o_rank, int d_model, int o_dtype) {
  if (M < 0 || H < 1 || head_dim < 1 || groups < 1 || o_rank < 1 || d_model < 1) return 0;
  const int64_t hd = int64_t(H) * head_dim;
  if (hd % groups != 0 || (hd / groups) % 128 != 0 || (int64_t(groups) * o_rank) % 128 != 0) return 0;
  const OPlan o = o_plan(M, groups, o_rank, hd / groups, d_model, o_dtype == CSA_F32);
  return (o.r + o.y) * sizeof(float);
}

int csa_out_proj(const void* o, int o_dtype, const void* wo_a, const void* wo_b, int M, int H, int head_dim,
                 int groups, int o_rank, int d_model, void* y, int y_dtype, void* ws, size_t ws_bytes,
                 hipStream_t stream) {
  if (!dtype_ok(o_dtype) || !dtype_ok(y_dtype)) return CSA_ERR_INVALID_ARG;
  if (M < 0 || H < 1 || head_dim < 1 || groups < 1 || o_rank < 1 || d_model < 1) return CSA_ERR_INVALID_ARG;
  const int64_t hd = int64_t(H) * head_dim;
  if (hd % groups != 0) return CSA_ERR_INVALID_ARG;
  const int64_t kg = hd / groups, kb = int64_t(groups) * o_rank;
  if (kg > INT32_MAX || kb > INT32_MAX) return CSA_ERR_UNSUPPORTED;
  if (!proj_dims_ok(M, o_rank, int(kg)) || !proj_dims_ok(M, d_model, int(kb))) return CSA_ERR_UNSUPPORTED;
  if (int64_t((o_rank + 127) / 128) * groups > 0x7fffffff || int64_t(M) > 65535 * 32) return CSA_ERR_UNSUPPORTED;
  if (M == 0) return CSA_OK;  // no token: nothing is read or written, the pointers may be NULL
  if (!o || !wo_a || !wo_b || !y) return CSA_ERR_INVALID_ARG;
  if (!aligned16(o) || !aligned16(wo_a) || !aligned16(wo_b) || !aligned16(y)) return CSA_ERR_INVALID_ARG;
  const size_t need = csa_out_proj_workspace_size(M, H, head_dim, groups, o_rank, d_model, o_dtype);
  if (need > 0 && (ws == nullptr || ws_bytes < need)) return CSA_ERR_WORKSPACE;
  if (need > 0 && !aligned16(ws)) return CSA_ERR_INVALID_ARG;
  const OPlan pl = o_plan(M, groups, o_rank, kg, d_model, o_dtype == CSA_F32);
  float* r = static_cast<float*>(ws);
  float* yp = r + pl.r;
  // one down-projection per group of heads (K-chunk partials)
  csa::ProjArgs ga{o, o_dtype, hd, kg, wo_a, int64_t(o_rank) * kg, r, CSA_F32, kb, o_rank, M, o_rank, int(kg),
                   groups, 1, 0, pl.pa.kc, pl.pa.ks, r, int64_t(M) * kb};
  if (csa::launch_proj_gemm(ga, stream) != hipSuccess) return CSA_ERR_HIP;
  // the concatenated group results (summing the partials) back to the model width
  csa::ProjArgs gb{r, CSA_F32, kb, 0, wo_b, 0, y, y_dtype, d_model, 0, M, d_model, int(kb), 1, pl.pa.ks,
                   int64_t(M) * kb, pl.pb.kc, pl.pb.ks, yp, int64_t(M) * d_model};
  if (csa::launch_proj_gemm(gb, stream) != hipSuccess) return CSA_ERR_HIP;
  if (pl.pb.ks > 1 && csa::launch_proj_reduce(gb, stream) != hipSuccess) return CSA_ERR_HIP;
  return CSA_OK;
}

}  // extern "C"
