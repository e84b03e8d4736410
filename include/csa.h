/*
 * csa.h -- C ABI of the CSA / HCA compressed-KV attention path for gfx950.
 *
 * Compressed Sparse Attention (CSA) pools every completed group of `ratio`
 * tokens into one compressed entry, scores all visible entries with a
 * many-head indexer, keeps the top-k and runs one softmax over a sliding
 * window plus the kept entries, with a per-head sink.  Heavily Compressed
 * Attention (HCA) uses a larger ratio and attends to every visible entry.
 *
 * Sources, cited by page title and section:
 *   [V4-Flash walkthrough] "DeepSeek-V4-Flash 架构：一个 token 的旅程"
 *       (hs-black.github.io/posts/deepseek-v4-flash/)
 *   [V4.1 lab]  "Lab tổng hợp DeepSeek-V4.1-Flash" (openarchlab.com)
 *   [LLM Atlas] "LLM Atlas: DeepSeek" (llm-atlas.k1412.top/deepseek/), §19
 *
 * Conventions shared by every entry point
 *   - Pointers are DEVICE pointers unless stated otherwise; the caller owns
 *     every buffer (inputs, outputs, workspace).  The library never
 *     allocates, frees or synchronises; all work is enqueued on `stream`
 *     (NULL = the default stream) in call order.
 *   - Tensors are dense, row-major, innermost dimension contiguous, 16-byte
 *     aligned.  bf16 tensors hold raw bfloat16 bit patterns.
 *   - dtype codes: CSA_F32 (float32) and CSA_BF16 (bfloat16).  Weights w,
 *     sink, gamma and scores are always float32.  Arithmetic is float32
 *     (bf16 x bf16 products accumulate in float32 on the matrix cores).
 *   - Positions are 0-based token indices.  RoPE rotates interleaved pairs
 *     (2i, 2i+1) of the trailing `rope_dim` channels by
 *     pos * rope_base^(-2i/rope_dim); the angle is formed and reduced in
 *     double precision.  A compressed entry e of ratio r sits at position
 *     e*r.
 *   - Return value: CSA_OK, or a negative CSA_ERR_* code.  Arguments are
 *     validated on the host before any HIP call, so a rejected call has no
 *     side effect.  Index values read from device memory (positions,
 *     selections) are bounds-checked in the kernels: out-of-range values are
 *     skipped, never dereferenced.
 */
#ifndef CSA_H_
#define CSA_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { CSA_F32 = 0, CSA_BF16 = 1 };

enum {
  CSA_OK = 0,
  CSA_ERR_INVALID_ARG = -1,   /* null pointer, bad size, inconsistent shapes   */
  CSA_ERR_UNSUPPORTED = -2,   /* shape / dtype combination not compiled        */
  CSA_ERR_HIP = -3,           /* a HIP launch or runtime call failed           */
  CSA_ERR_WORKSPACE = -4      /* ws_bytes below the matching *_workspace_size  */
};

/* Static, human-readable name of a status code. */
const char* csa_status_string(int status);

/* Library version, major*10000 + minor*100 + patch. */
int csa_version(void);

/*
 * csa_compress -- build compressed entries from per-token rows.
 *
 * [V4-Flash walkthrough] "压缩是逐通道的 learned pooling" and
 * "一个通道，逐项算出压缩结果": entry e pools the current group, tokens
 * [e*r, (e+1)*r) read from (kv, gate), and, when `overlap` is set, the
 * previous group [(e-1)*r, e*r) read from (kv_prev, gate_prev).  For e == 0
 * the previous group does not exist (gate -inf, weight 0): its rows are not
 * read.  Per channel c the gates go through a softmax over the candidates,
 * y[c] = sum_j p_j[c] * v_j[c]; then y <- gamma * y / sqrt(mean(y^2) + eps);
 * then RoPE on the trailing rope_dim channels at position e*r.
 * "压缩条目必须等整组完成后才可见": an entry exists once its group is complete.
 *
 *   kv, gate          [B, *, D] per-token rows (in_dtype); sequence b starts
 *                     at element b*in_bstride; token rows are D elements apart.
 *   kv_prev, gate_prev rows of the previous-group role, same layout; NULL
 *                     means "same as kv / gate".
 *   gamma             [D] float32 RMSNorm weight.
 *   ratio >= 1, overlap in {0,1}, rope_dim even and <= D, eps >= 0.
 *   out               [B, out_cap, D] (out_dtype); entry e of sequence b is
 *                     written at out + (b*out_bstride + e*D) elements.
 *
 *   Span mode (pos == NULL): row j of each sequence holds token tok0 + j,
 *     0 <= j < T.  Entries e0 .. e0+n_entries-1 are written for every
 *     sequence; their tokens must lie in [tok0, tok0+T) and
 *     e0 + n_entries <= out_cap.
 *   Ring mode (pos != NULL, [B] int32): the T rows of a sequence are a ring,
 *     token t at row t % T, with T >= (1+overlap)*ratio.  Sequence b emits
 *     entry pos[b]/ratio iff (pos[b]+1) % ratio == 0 (its group just
 *     completed) and that entry is < out_cap; otherwise it writes nothing.
 *     tok0, e0 and n_entries are ignored.  This is the decode-time append.
 *
 *   ws, ws_bytes      device workspace of csa_compress_workspace_size(entries,
 *                     D, ratio, overlap) bytes, entries = B in ring mode and
 *                     B*n_entries in span mode; 16-byte aligned, caller-owned,
 *                     may be NULL when that size is 0 (it is non-zero only for
 *                     long candidate lists of at most 256 entries, whose
 *                     candidates are split over several workgroups).  It must
 *                     hold zeros before its first use; every call leaves it
 *                     ready for the next (its per-entry counters back at zero).
 *                     Calls that overlap in time must not share one workspace.
 *                     Returns CSA_ERR_WORKSPACE when too small,
 *                     CSA_ERR_INVALID_ARG when misaligned.
 */
size_t csa_compress_workspace_size(int64_t entries, int D, int ratio, int overlap);
int csa_compress(const void* kv, const void* gate, const void* kv_prev, const void* gate_prev,
                 int in_dtype, const float* gamma,
                 int B, int T, int64_t in_bstride, int D,
                 int ratio, int overlap, int rope_dim, float rope_base, float eps,
                 int tok0, int e0, int n_entries, const int* pos,
                 void* out, int out_dtype, int64_t out_bstride, int out_cap,
                 void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * csa_compress_jobs -- several independent csa_compress calls, launched
 * together.
 *
 * A decode step appends to two caches (KV entries and index keys), each one
 * csa_compress call whose time is mostly one chain of memory latencies; run
 * as one launch, the chains overlap.  Every job holds exactly the arguments
 * of one csa_compress call (same meaning, same validation, same workspace
 * rules) and its results are bit-identical to that call's.  Jobs must be
 * independent: no job may write memory another job reads or writes.
 *
 *   jobs     HOST array of n_jobs descriptors (read during the call only)
 *   n_jobs   0 .. CSA_MAX_COMPRESS_JOBS
 * Every job is validated before anything is launched: a rejected call
 * (the first failing job's status) launches nothing.  Jobs that share a
 * kernel configuration (one workgroup per entry, the same channels per lane
 * and input dtype) run in one kernel, at most four per kernel; the others run
 * one kernel each, in order, on `stream`.
 */
#define CSA_MAX_COMPRESS_JOBS 16
typedef struct csa_compress_job {
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
  int tok0, e0, n_entries;
  const int* pos;
  void* out;
  int out_dtype;
  int64_t out_bstride;
  int out_cap;
  void* ws;
  size_t ws_bytes;
} csa_compress_job;
int csa_compress_jobs(const csa_compress_job* jobs, int n_jobs, hipStream_t stream);

/*
 * csa_index_score -- indexer scores of every compressed entry.
 *
 * [V4-Flash walkthrough] "少读 KV 之前，Indexer 仍要给历史打分": H_I heads of
 * dim D_I score one shared D_I-wide index cache with signed per-head weights
 * w (w already carries the 1/sqrt(D_I)/sqrt(H_I) scale).  [V4.1 lab]
 * "3 Giải pháp": a ReLU acts on every head's dot product.
 *   scores[b,s,e] = sum_h w[b,s,h] * max(0, q_idx[b,s,h,:] . idx_cache[b,e,:])
 * for e < n_vis = min((pos[b,s]+1)/ratio, Ncap)  ("压缩条目必须等整组完成后才可见"),
 * and -inf for n_vis <= e < Ncap.
 *
 *   q_idx     [B, S, H_I, D_I] (dtype);  w [B, S, H_I] float32
 *   idx_cache [B, Ncap, D_I]   (dtype);  pos [B, S] int32
 *   scores    [B, S, Ncap]     float32 (written in full)
 * Matrix-core path: dtype CSA_BF16, H_I == 64, D_I == 128.  Other shapes run
 * a vector-ALU path (D_I <= 1024, H_I <= 1024).
 */
int csa_index_score(const void* q_idx, const float* w, const void* idx_cache, int dtype,
                    const int* pos, int B, int S, int H_I, int D_I, int Ncap, int ratio,
                    float* scores, hipStream_t stream);

/*
 * csa_topk -- the k best entries of every score row.
 *
 * [V4-Flash walkthrough] "少读 KV 之前，Indexer 仍要给历史打分" (top-k picks
 * what the main attention reads); [LLM Atlas] §19 (k = 512 for Flash).
 * Row r considers entries j < n_valid[r] (all N when n_valid is NULL) whose
 * score is not -inf; it keeps the k largest, ties going to the lower index.
 * idx[r, :] receives the kept indices in ascending order, padded with -1 when
 * fewer than k qualify.  Scores must not be NaN.
 *
 *   scores [R, N] float32; n_valid [R] int32 or NULL; idx [R, k] int32
 *   1 <= k <= 4096.  ws: device workspace of csa_topk_workspace_size(R,N,k)
 *   bytes (may be NULL when that size is 0).
 */
size_t csa_topk_workspace_size(int R, int N, int k);
int csa_topk(const float* scores, const int* n_valid, int R, int N, int k, int* idx,
             void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * csa_sparse_attn -- CSA joint-softmax attention with a sink.
 *
 * [V4-Flash walkthrough] "局部和压缩记忆，共用一次归一化": the window rows and
 * the selected compressed rows form one candidate set under one softmax; the
 * per-head sink adds exp(sink[h]) to the denominator and has no value.
 * "输出投影也分组，并且降低中间维度": the output is rotated back
 * (inverse RoPE at the query position).  [V4.1 lab] "3 Giải pháp": all query
 * heads share one K/V head; K and V are the same row.
 *   For query (b,s) at p = pos[b,s] and head h, over candidates j:
 *     window rows: positions max(0, p-window+1) .. p, read from
 *                  win + (b*Wcap + position % Wcap)*D   (a ring of Wcap >= window rows)
 *     selected:    cmp + (b*Ncap + e)*D for e = idx[b,s,i], 0 <= e < Ncap
 *                  (-1 and out-of-range entries are skipped)
 *     l_j = scale * q[b,s,h,:] . row_j;   m = max(max_j l_j, sink[h])
 *     o = sum_j e^(l_j-m) row_j / (sum_j e^(l_j-m) + e^(sink[h]-m))
 *     out[b,s,h,:] = inverse RoPE of o at position p
 *
 *   q [B,S,H,D] (dtype), cmp [B,Ncap,D] (dtype), idx [B,S,k] int32,
 *   win [B,Wcap,D] (dtype), pos [B,S] int32, sink [H] float32,
 *   out [B,S,H,D] (out_dtype).  A prefill passes its per-token window rows
 *   with Wcap >= the largest position + 1.
 * Matrix-core path: dtype CSA_BF16, H == 64, D == 512.  Other shapes run a
 * vector-ALU path (D <= 1024).  ws: csa_sparse_attn_workspace_size bytes,
 * 16-byte aligned, caller-owned (device memory; may be null when the size
 * is 0): split partials for few queries, one recompute flag per query for
 * many.  Returns CSA_ERR_WORKSPACE when too small, CSA_ERR_INVALID_ARG when
 * misaligned.
 */
size_t csa_sparse_attn_workspace_size(int B, int S, int H, int D, int k, int window);
int csa_sparse_attn(const void* q, const void* cmp, int Ncap, const int* idx, int k,
                    const void* win, int Wcap, int window, const int* pos, const float* sink,
                    int dtype, float scale, int rope_dim, float rope_base,
                    int B, int S, int H, int D, void* out, int out_dtype,
                    void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * hca_attn -- HCA attention: the window plus EVERY visible compressed entry.
 *
 * [LLM Atlas] §19: HCA keeps all compressed entries and takes no top-k.
 * [V4-Flash walkthrough] "长上下文时，先数真正访问的条目": its read count
 * grows with the context.  Same as csa_sparse_attn with the selection
 * replaced by entries 0 .. n_vis-1, n_vis = min((pos+1)/ratio, Ncap).
 * ws: hca_attn_workspace_size bytes (as for csa_sparse_attn).
 */
size_t hca_attn_workspace_size(int B, int S, int H, int D, int Ncap, int window);
int hca_attn(const void* q, const void* cmp, int Ncap, int ratio,
             const void* win, int Wcap, int window, const int* pos, const float* sink,
             int dtype, float scale, int rope_dim, float rope_base,
             int B, int S, int H, int D, void* out, int out_dtype,
             void* ws, size_t ws_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* CSA_H_ */
