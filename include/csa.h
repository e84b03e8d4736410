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
 *     aligned.  bf16 tensors hold raw bfloat16 bit patterns.  On the shapes
 *     that run the matrix-core or lane kernels (named at each entry point) a
 *     tensor that is not 16-byte aligned is rejected with
 *     CSA_ERR_INVALID_ARG; it is never sent down a slower path.
 *   - dtype codes: CSA_F32 (float32) and CSA_BF16 (bfloat16).  Weights w,
 *     sink, gamma and scores are always float32.  Arithmetic is float32
 *     (bf16 x bf16 products accumulate in float32 on the matrix cores).
 *   - Positions are 0-based token indices.  RoPE rotates interleaved pairs
 *     (2i, 2i+1) of the trailing `rope_dim` channels by
 *     pos * rope_base^(-2i/rope_dim); the angle is formed and reduced in
 *     double precision.  A compressed entry e of ratio r sits at position
 *     e*r.
 *   - A call with no work returns CSA_OK after checking its scalar arguments,
 *     reads and writes nothing and makes no HIP call; its pointers may then
 *     be NULL (as for empty tensors), the page table included.  No work
 *     means: csa_compress* builds no entry (B = 0, or n_entries = 0 without
 *     pos); csa_index_score* has B*S = 0 or no cache row; csa_topk* has
 *     R = 0; the attention calls have B*S = 0; csa_kv4_quantize has
 *     rows = 0; the projections have M = 0.  csa_topk* also accepts NULL
 *     scores when N = 0 (every selection is then -1).
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

/* CSA_KV4: the quantised compressed-KV row format (FP4 E2M1 latent, FP8 E4M3
 * RoPE tail, one power-of-two scale per 32 channels; see csa_kv4_quantize).
 * It is a cache format only: csa_compress may write it, csa_sparse_attn and
 * hca_attn read it (their queries and window rows stay bf16). */
enum { CSA_F32 = 0, CSA_BF16 = 1, CSA_KV4 = 2 };

enum {
  CSA_OK = 0,
  CSA_ERR_INVALID_ARG = -1,   /* null pointer, bad size, inconsistent shapes   */
  CSA_ERR_UNSUPPORTED = -2,   /* shape / dtype combination not compiled        */
  CSA_ERR_HIP = -3,           /* a HIP launch or runtime call failed           */
  CSA_ERR_WORKSPACE = -4,     /* ws_bytes below the matching *_workspace_size  */
  CSA_ERR_NO_PAGES = -5       /* a page pool has too few free pages            */
};

/* Static, human-readable name of a status code. */
const char* csa_status_string(int status);

/* Library version, major*10000 + minor*100 + patch. */
int csa_version(void);

/*
 * csa_kv4_row_bytes / csa_kv4_quantize -- the quantised compressed-KV cache.
 *
 * [V4.1 lab] "3 Giải pháp": the cache budget is priced with FP4 E2M1 for the
 * latent and FP8 E4M3 for the RoPE tail; [LLM Atlas] "FP8 训练真正难在哪":
 * low precision takes fine-grained scaling.  The block scaling and the byte
 * layout are this library's reading (the pages give neither):
 *   row = [latent codes: (D-rope_dim)/2 bytes, two per byte, even channel in
 *          the low nibble] [tail codes: rope_dim bytes] [one scale byte per
 *          32 channels, latent blocks first: the block scale is 2^(byte-127),
 *          the smallest power of two that brings the block's largest
 *          magnitude within 6 (E2M1) or 448 (E4M3)] [zeros to 16 bytes];
 *   elements round to the nearest code, ties to the even code, and a value
 *   rounding to zero keeps its sign.
 * D = 512 with a 64-wide tail: 304 bytes per row (1024 in bf16).
 *
 * csa_kv4_row_bytes returns the row size, or 0 when D or rope_dim is not a
 * multiple of 32 (the format needs whole blocks).
 * csa_kv4_quantize writes rows [rows, row_bytes] (out, 16-byte aligned) from
 * x [rows, D] (x_dtype CSA_F32 or CSA_BF16).
 */
size_t csa_kv4_row_bytes(int D, int rope_dim);
int csa_kv4_quantize(const void* x, int x_dtype, int64_t rows, int D, int rope_dim, void* out,
                     hipStream_t stream);

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
 *                     written at out + (b*out_bstride + e*D) elements.  With
 *                     out_dtype CSA_KV4 the entry is written quantised:
 *                     out_bstride counts bytes (a multiple of 16) and entry e
 *                     is the row at out + b*out_bstride + e*csa_kv4_row_bytes
 *                     bytes (D and rope_dim multiples of 32).
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
 *                     candidates are split over several workgroups).  Its
 *                     first 1 KiB holds 256 per-entry arrival counters at a
 *                     fixed place for every call shape; the partial states
 *                     follow.  It must hold zeros before its first use; every
 *                     call leaves the counters back at zero, so one workspace
 *                     of the largest size needed may serve calls of any batch,
 *                     width and ratio in turn.  Calls that overlap in time
 *                     must not share one workspace.
 *                     Returns CSA_ERR_WORKSPACE when too small,
 *                     CSA_ERR_INVALID_ARG when misaligned.
 *   Lane kernel (D a multiple of 128): kv, gate, kv_prev, gate_prev and out
 *   must be 16-byte aligned and their sequence strides a multiple of 16
 *   bytes, else CSA_ERR_INVALID_ARG.
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
 * Matrix-core path: dtype CSA_BF16, H_I == 64, D_I == 128; q_idx, idx_cache
 * and scores must then be 16-byte aligned (else CSA_ERR_INVALID_ARG).  Other
 * shapes run a vector-ALU path (D_I <= 1024, H_I <= 1024).
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
 * csa_topk_noalloc -- csa_topk without a caller workspace, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).
 *
 * Same arguments, results and validation as csa_topk, bit for bit.  Rows of
 * at most 16,384 positions need no scratch; longer rows keep their chunk
 * candidates in a static device array of CSA_TOPK_NOALLOC_SCRATCH_BYTES
 * (16 MiB) that every device the library runs on holds until the process
 * ends (its address is looked up on the first call on each device).  Calls
 * needing more than that (csa_topk_workspace_size(R, N, k) above the limit,
 * e.g. 32 rows of 262,144 positions at k = 1024 fit, 64 such rows do not)
 * return CSA_ERR_WORKSPACE.  The call allocates and frees nothing.  All calls
 * on one device share the one array: calls that may overlap in time on one
 * device (different streams without ordering between them) race and must
 * not be issued.  Nothing in the array needs to start at zero.
 */
#define CSA_TOPK_NOALLOC_SCRATCH_BYTES (16u << 20)
int csa_topk_noalloc(const float* scores, const int* n_valid, int R, int N, int k, int* idx,
                     hipStream_t stream);

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
 *   with Wcap >= the largest position + 1.  dtype CSA_KV4: q and win are
 *   bf16 and cmp holds quantised rows [B, Ncap, csa_kv4_row_bytes(D,
 *   rope_dim)] bytes, dequantised exactly to bf16 on the way into the
 *   products (D and rope_dim multiples of 32).
 * Matrix-core path: dtype CSA_BF16, H == 64, D == 512; q, cmp, win and out
 * must then be 16-byte aligned (else CSA_ERR_INVALID_ARG).  Other shapes run
 * a vector-ALU path (D <= 1024).  ws: csa_sparse_attn_workspace_size bytes,
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

/*
 * Paged, variable-length compressed caches.
 *
 * [LLM Atlas] §19 "V4 / HETEROGENEOUS STATE MACHINE": real serving depends on
 * the batch, the distribution of sequence lengths, quantisation and the page
 * allocator.  A paged cache keeps the rows of all sequences in one pool of
 * pages of page_rows rows each (rows as in the contiguous layout: D elements
 * of the cache dtype, or csa_kv4_row_bytes bytes); a block table maps
 * logical page j of sequence b to a pool page:
 *   entry e of sequence b -> pool row pages[b*max_pages + e/page_rows]*page_rows
 *                                      + e % page_rows
 * so sequences grow page by page, independently of each other.
 *
 *   pages       DEVICE int32 [B, max_pages]; -1 marks a page not allocated.
 *               Entries the kernels reach must be pool pages in
 *               [0, pool_pages).  Others are the caller's error and never
 *               leave the pool: an appended entry is not written, an attended
 *               row is left out, and an index score is -inf on the vector
 *               path but, on the matrix-core kernels, the score of the pool's
 *               first page's row (finite, meaningless).
 *   page_rows   a power of two >= 64 (the indexer's waves read 64 rows at a time).
 *   pool_pages  pages in the pool.
 * The logical capacity of a sequence is Ncap = max_pages * page_rows; score
 * rows stay [B, S, Ncap] in logical order and top-k is unchanged.
 */
typedef struct csa_page_table {
  const int* pages;
  int max_pages;
  int page_rows;
  int pool_pages;
} csa_page_table;

/* csa_compress_jobs with outputs in paged caches: jobs[i] holds the
 * arguments of one csa_compress call with out = its pool (out_bstride and
 * out_cap are taken from tables[i]), and all n_jobs (0 .. CSA_MAX_COMPRESS_JOBS)
 * run in one launch, e.g. the KV and index-key appends of a decode step.
 * Ring mode appends entry pos/r of sequence b at its pool row; span mode
 * writes entries e0 .. e0+n-1.  Host arrays, read before the call returns. */
int csa_compress_paged(const csa_compress_job* jobs, const csa_page_table* tables, int n_jobs, hipStream_t stream);

/* csa_index_score over a paged index-key cache (idx_pool: the pool; Ncap =
 * max_pages*page_rows).  Matrix-core shapes take the streaming kernel. */
int csa_index_score_paged(const void* q_idx, const float* w, const void* idx_pool, int dtype, const int* pos,
                          int B, int S, int H_I, int D_I, const csa_page_table* pages, int ratio, float* scores,
                          hipStream_t stream);

/* csa_sparse_attn / hca_attn over a paged compressed cache (cmp_pool: the
 * pool, bf16 rows or, with dtype CSA_KV4, quantised rows).  Selections are
 * logical entries.  Workspace: csa_sparse_attn_workspace_size /
 * hca_attn_workspace_size (with Ncap = max_pages*page_rows) cover the paged
 * plans. */
int csa_sparse_attn_paged(const void* q, const void* cmp_pool, const csa_page_table* pages, const int* idx, int k,
                          const void* win, int Wcap, int window, const int* pos, const float* sink, int dtype,
                          float scale, int rope_dim, float rope_base, int B, int S, int H, int D, void* out,
                          int out_dtype, void* ws, size_t ws_bytes, hipStream_t stream);
int hca_attn_paged(const void* q, const void* cmp_pool, const csa_page_table* pages, int ratio, const void* win,
                   int Wcap, int window, const int* pos, const float* sink, int dtype, float scale, int rope_dim,
                   float rope_base, int B, int S, int H, int D, void* out, int out_dtype, void* ws,
                   size_t ws_bytes, hipStream_t stream);

/*
 * csa_page_pool -- the page allocator behind paged caches (host memory only;
 * the device pool itself is the caller's allocation).
 *
 * create: a pool of n_pages free pages (NULL when n_pages < 1 or out of
 *   host memory); pages are handed out lowest-numbered first while the pool
 *   is fresh, then most recently released first.
 * alloc: n pages into the HOST array pages, or CSA_ERR_NO_PAGES (nothing
 *   taken).  release: gives n pages back; every page must be in use and
 *   named once, else CSA_ERR_INVALID_ARG and nothing is released.
 * csa_page_table_reserve: makes a sequence's HOST table row (max_pages
 *   entries, -1 = none) cover n_entries entries, allocating only the missing
 *   pages (all or nothing).  csa_page_table_release frees every page of a row
 *   and sets it to -1.  Upload the table to the device before the kernels
 *   read it.  All calls are thread-safe.
 */
typedef struct csa_page_pool csa_page_pool;
csa_page_pool* csa_page_pool_create(int n_pages);
void csa_page_pool_destroy(csa_page_pool* pool);
int csa_page_pool_available(csa_page_pool* pool);
int csa_page_pool_alloc(csa_page_pool* pool, int n, int* pages);
int csa_page_pool_release(csa_page_pool* pool, int n, const int* pages);
int csa_page_table_reserve(csa_page_pool* pool, int* row, int max_pages, int page_rows, int64_t n_entries);
int csa_page_table_release(csa_page_pool* pool, int* row, int max_pages);

/*
 * csa_q_proj -- the low-rank query path in front of the attention.
 *
 * [V4-Flash walkthrough] "低秩 Q：两次矩阵乘法接起来": for every token m,
 *   qr   = RMSNorm(x[m] . wq_a^T) * gamma_q          (latent of q_rank)
 *   q[m] = qr . wq_b^T viewed as H heads of head_dim
 *   every head divided by its own sqrt(mean(q^2) + eps) (no gain)
 *   RoPE on the trailing rope_dim dims of every head at position pos[m]
 * (the Flash widths: d_model 4096, q_rank 1024, 64 heads of 512, RoPE 64).
 * The latent's RMSNorm carries the learned gain gamma_q (a reading; the page
 * calls a normalisation layer there).
 *
 *   x      [M, d_model] bf16 (token rows; M = B*S)
 *   wq_a   [q_rank, d_model] bf16;  gamma_q [q_rank] float32
 *   wq_b   [H*head_dim, q_rank] bf16
 *   pos    [M] int32 (may be NULL when rope_dim == 0)
 *   q      [M, H, head_dim] bf16 -- the layout csa_sparse_attn / hca_attn read
 *   ws     device workspace of csa_q_proj_workspace_size(M, d_model, q_rank,
 *          H, head_dim) bytes (fp32 partial sums of the products over K
 *          chunks, the normalised latent), 16-byte aligned, caller-owned.
 * Requires d_model and q_rank multiples of 128, H*head_dim a multiple of 16,
 * q_rank <= 16384, and 16-byte aligned x, wq_a, wq_b, q (else
 * CSA_ERR_UNSUPPORTED / CSA_ERR_INVALID_ARG).  The matrix products run on the
 * matrix cores with fp32 accumulation; the fp32 latent enters the second
 * product as a bf16 head plus a bf16 remainder (about 16 significant bits).
 */
size_t csa_q_proj_workspace_size(int M, int d_model, int q_rank, int H, int head_dim);
int csa_q_proj(const void* x, const void* wq_a, const float* gamma_q, const void* wq_b, const int* pos,
               int M, int d_model, int q_rank, int H, int head_dim, int rope_dim, float rope_base,
               float eps, void* q, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * csa_out_proj -- the grouped output projection behind the attention.
 *
 * [V4-Flash walkthrough] "输出投影也分组，并且降低中间维度": the attention
 * output o (already rotated back by csa_sparse_attn / hca_attn) is viewed as
 * `groups` groups of H*head_dim/groups values (group g = heads
 * g*H/groups .. (g+1)*H/groups - 1); group g goes through its own
 * down-projection wo_a[g] (o_rank rows), i.e. einsum("bsgd,grd->bsgr"); the
 * concatenated group results go through wo_b back to d_model
 * (the Flash widths: 8 groups of 8 heads, o_rank 1024, d_model 4096).
 *
 *   o      [M, H, head_dim] (o_dtype: CSA_BF16, or CSA_F32 which enters the
 *          products as a bf16 head plus a bf16 remainder)
 *   wo_a   [groups, o_rank, H*head_dim/groups] bf16
 *   wo_b   [d_model, groups*o_rank] bf16
 *   y      [M, d_model] (y_dtype)
 *   ws     device workspace of csa_out_proj_workspace_size(M, H, head_dim,
 *          groups, o_rank, d_model, o_dtype) bytes (fp32 partial sums of the
 *          group results and of y over K chunks), 16-byte aligned,
 *          caller-owned.
 * Requires H*head_dim/groups and groups*o_rank multiples of 128, o_rank and
 * d_model multiples of 16, 16-byte aligned o, wo_a, wo_b, y.
 */
size_t csa_out_proj_workspace_size(int M, int H, int head_dim, int groups, int o_rank, int d_model, int o_dtype);
int csa_out_proj(const void* o, int o_dtype, const void* wo_a, const void* wo_b, int M, int H, int head_dim,
                 int groups, int o_rank, int d_model, void* y, int y_dtype, void* ws, size_t ws_bytes,
                 hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* CSA_H_ */
