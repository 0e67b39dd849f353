/*
 * infv2.h -- C ABI of the InfLLM-V2 sparse-attention forward path on MI355X.
 *
 * The method: InfLLM-V2 dense-sparse switchable attention, as described on
 *  - the papernotes.org note "InfLLM-V2: Dense-Sparse Switchable Attention for
 *    Seamless Short-to-Long Adaptation", 方法详解 > 关键设计 2-4 (key designs 2-4);
 *  - the paperlayer.ai summary of arXiv 2509.24663v1, "A IMPLEMENTATION DETAIL";
 *  - the OpenBMB blog "技术Blog-4 | 新一代InfLLM：可训练的稀疏注意力机制",
 *    动态上下文块选择 (semantic kernels, top-k sharing, efficient top-k).
 *
 * Conventions for every entry point
 *  - All pointers are DEVICE pointers except `prob` (host).  Buffers are
 *    row-major and contiguous with the layouts stated per call; every device
 *    pointer must be 16-byte aligned.
 *  - The caller owns and frees every buffer, workspaces included.  The
 *    library keeps no state besides a thread-local error string (and, for
 *    infv2_sparse_attn_noalloc alone, one static scratch array per GPU): it
 *    never allocates, never synchronises and never writes an input.
 *  - All work is enqueued on `stream` (a hipStream_t passed as void*; NULL is
 *    the default stream).  Calls return once the work is enqueued.
 *  - Return value: INFV2_OK, or a negative status; infv2_last_error() then
 *    holds a message for the calling thread.  Nothing is enqueued when a
 *    call returns an argument, support or workspace error.
 *  - Entry points are reentrant; no C++ exception crosses this boundary.
 *
 * Notation (the pages'): B block size; l_C1, s_C1 stage-1 kernel length and
 * stride; l, s stage-3 max-pool length and stride (in kernels); k top-k; N_init,
 * N_local; G query heads per KV group; h_q = G*h_kv; d head dimension.
 */
#ifndef INFV2_H
#define INFV2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  INFV2_OK = 0,
  INFV2_E_ARG = -1,          /* null/misaligned pointer, inconsistent sizes   */
  INFV2_E_UNSUPPORTED = -2,  /* valid for the method, no kernel instance      */
  INFV2_E_WORKSPACE = -3,    /* workspace too small                           */
  INFV2_E_HIP = -4           /* a HIP launch failed (message holds the error) */
};

enum { INFV2_BF16 = 0, INFV2_F32 = 1 };

/* One attention layer call.  Query token t of a sequence sits at absolute
 * position p = q_pos0 + t (prefill: q_pos0 = 0, n_q = n_kv; decode:
 * q_pos0 = L-1, n_q = 1, n_kv = L, the cache length INCLUDING the new token).
 * Head h belongs to KV group g = h / G (the G heads of a group are adjacent). */
typedef struct infv2_problem {
  int32_t batch;             /* b: sequences                                   */
  int32_t n_q;               /* query tokens per sequence                      */
  int32_t q_pos0;            /* absolute position of query token 0             */
  int32_t n_kv;              /* keys per sequence (q_pos0 + n_q <= n_kv)       */
  int32_t h_kv;              /* KV heads (groups)                              */
  int32_t G;                 /* query heads per group                          */
  int32_t d;                 /* head dimension                                 */
  int32_t B;                 /* KV block size                                  */
  int32_t l_C1, s_C1;        /* stage-1 kernel length / stride (tokens)        */
  int32_t l, s;              /* stage-3 max-pool length / stride (kernels)     */
  int32_t k;                 /* top-k blocks besides init and local            */
  int32_t N_init, N_local;   /* always-attended initial / local blocks         */
  int32_t dtype;             /* INFV2_BF16 or INFV2_F32: Q, K, V, K^C1 and O   */
  float scale;               /* softmax scale; 0 selects 1/sqrt(d)             */
  int64_t kv_cap;            /* token rows allocated in K and V; 0 -> n_kv     */
  int64_t c1_cap;            /* kernel rows allocated in K^C1; 0 -> n_C1       */
  int64_t c2_cap;            /* coarse kernel rows in K^C2; 0 -> n_C2          */
  int32_t lse_approx;        /* 1: estimate the stage-1 softmax normaliser from
                                coarse kernels (see infv2_compress_k2); 0: exact */
} infv2_problem;

/* Derived sizes.  n_C1 = floor((n_kv - l_C1)/s_C1) + 1 complete kernels
 * (0 if n_kv < l_C1); n_C2 the same for the coarse kernels (l_C2 = 4 l_C1,
 * s_C2 = 4 s_C1); n_blk = ceil(n_kv / B); budget = N_init + N_local + k. */
int32_t infv2_n_kernels(const infv2_problem* prob);
int32_t infv2_n_coarse_kernels(const infv2_problem* prob);
int32_t infv2_n_blocks(const infv2_problem* prob);
int32_t infv2_budget(const infv2_problem* prob);

/* 1 when ceil(n_kv/B) <= N_init + N_local + k: every causal block is in the
 * budget and the sparse path equals dense causal attention (papernotes note,
 * 整体框架 flowchart; OpenBMB blog, 语义核: short inputs degrade to standard
 * attention).  0 otherwise, -1 on a bad argument. */
int infv2_use_dense(const infv2_problem* prob);

/* Checks that `prob` describes a problem the library can run (shapes, the
 * max-pool parameters l and s equal the count and stride of the kernels that
 * intersect a block, B a multiple of the attention key tile, batch x
 * min(n_q, 4) <= 65535 so that one launch grid dimension holds it, ...).
 * Returns INFV2_OK, INFV2_E_ARG or INFV2_E_UNSUPPORTED; enqueues nothing. */
int infv2_check_problem(const infv2_problem* prob);

/* Stage 1 (papernotes note, 关键设计 3; OpenBMB blog, 语义核): mean-pool the keys
 * of each kernel,  K^C1[b][g][j][:] = (1/l_C1) * sum_{u<l_C1} K[b][j*s_C1+u][g][:],
 * for kernels j in [c1_begin, c1_end).  The sum is exact (compensated fp64)
 * and rounded once, to nearest even, to the I/O dtype.  Prefill passes
 * [0, n_C1); a decode step appends the kernels that the new tokens completed.
 *   K   : [batch][kv_cap][h_kv][d]   (input)
 *   Kc1 : [batch][h_kv][c1_cap][d]   (output rows c1_begin..c1_end-1 only)
 * Requires 0 <= c1_begin <= c1_end <= n_C1 <= c1_cap. */
int infv2_compress_k(const infv2_problem* prob, const void* K, void* Kc1,
                     int32_t c1_begin, int32_t c1_end, void* stream);

/* Coarse keys for the LSE approximation (papernotes note, 关键设计 4; OpenBMB
 * blog, 高效Top-K实现): K^C2[b][g][j][:] = (1/l_C2) * sum_{u<l_C2}
 * K[b][j*s_C2+u][g][:] with l_C2 = 4 l_C1 and s_C2 = 4 s_C1, for coarse
 * kernels j in [c2_begin, c2_end); exact sum, one rounding, as for K^C1.
 *   K   : [batch][kv_cap][h_kv][d]   (input)
 *   Kc2 : [batch][h_kv][c2_cap][d]   (output rows c2_begin..c2_end-1 only)
 * Requires 0 <= c2_begin <= c2_end <= n_C2 <= c2_cap. */
int infv2_compress_k2(const infv2_problem* prob, const void* K, void* Kc2,
                      int32_t c2_begin, int32_t c2_end, void* stream);

/* Stages 2-3 with the exact two-pass log-sum-exp (papernotes note, 关键设计 3
 * and 4; OpenBMB blog, 高效Top-K实现).  For query token t (position p), group g:
 *   z[h][j]     = scale * Q[b][t][h][:] . K^C1[b][g][j][:]   for visible j,
 *                 i.e. j*s_C1 + l_C1 - 1 <= p (a kernel is causal when its
 *                 last token is);
 *   S^C1[h][j]  = exp(z[h][j] - lse[h]),  lse[h] = log sum_j exp(z[h][j]);
 *   S^shared[j] = sum over the G heads of g of S^C1[h][j]   (kept on chip
 *                 unless the caller asks for it);
 *   S^cmp[blk]  = max of S^shared over the visible kernels that intersect
 *                 block blk (-inf when there is none).
 * With prob->lse_approx the normaliser is the coarse estimate instead (the
 * same pages, LSE approximation): lse[h] = log sum over the visible coarse
 * kernels j2 (j2*s_C2 + l_C2 - 1 <= p) of exp(scale * Q . K^C2[j2])
 * + ln(s_C2/s_C1); a token that sees no coarse kernel keeps the exact lse.
 * S^C1 is then exp(z - lse) in fp32 (+inf beyond the fp32 range).
 *   Q     : [batch][n_q][h_q][d]
 *   Kc1   : [batch][h_kv][c1_cap][d]  (rows 0..n_C1-1 valid)
 *   Kc2   : [batch][h_kv][c2_cap][d]  (rows 0..n_C2-1 valid) with
 *           lse_approx, else ignored (may be NULL)
 *   S_cmp : [batch][h_kv][n_q][n_blk] fp32 (output).  Entries for blocks
 *           0..floor(p/B) are written; entries after the query's own block are
 *           left untouched.
 *   S_shared : [batch][h_kv][n_q][n_C1] fp32 (optional output, may be NULL):
 *           S^shared[j] for every kernel, 0 for kernels the token does not
 *           see.  Asking for it costs one more fp32 write per kernel.
 *   ws    : workspace of infv2_block_scores_workspace(prob) bytes (may be
 *           NULL when that size is 0). */
size_t infv2_block_scores_workspace(const infv2_problem* prob);
int infv2_block_scores(const infv2_problem* prob, const void* Q, const void* Kc1,
                       const void* Kc2, float* S_cmp, float* S_shared, void* ws,
                       size_t ws_bytes, void* stream);

/* Block selection (papernotes note, 关键设计 2; OpenBMB blog, Top-K块共享):
 *   I(p) = I_init  u  I_local(p)  u  top-k(p),
 * I_init = {0..N_init-1}, I_local(p) = {b_p-N_local+1..b_p} with b_p = floor(p/B),
 * top-k = the k best remaining causal blocks by S^cmp; ties go to the lower
 * block index.  One set per (token, group), shared by the group's heads.
 *   S_cmp : [batch][h_kv][n_q][n_blk] fp32 (input, as written above)
 *   idx   : [batch][h_kv][n_q][budget] int32 (output): I(p) ascending, padded
 *           with -1; |I(p)| = min(b_p + 1, budget)
 *   n_sel : [batch][h_kv][n_q] int32 (output): |I(p)|. */
int infv2_topk_select(const infv2_problem* prob, const float* S_cmp, int32_t* idx,
                      int32_t* n_sel, void* stream);

/* Stages 2-3 and the block selection in one call (the same definitions as
 * infv2_block_scores followed by infv2_topk_select; OpenBMB blog,
 * 高效Top-K实现, fuses the top-k into the score computation as well).  idx
 * and n_sel are bitwise those of the two separate calls.  For decode-sized
 * problems (few query tokens, k <= 32) the pooling kernel keeps the k best
 * candidates of each group of 64 blocks and a small kernel merges those
 * lists, so S^cmp need not be stored.
 *   Kc2   : as in infv2_block_scores (with lse_approx).
 *   S_cmp : [batch][h_kv][n_q][n_blk] fp32 output as in infv2_block_scores,
 *           or NULL when the caller does not need the scores (they then live
 *           in the workspace where a path needs them).
 *   idx, n_sel : outputs as in infv2_topk_select.
 *   ws    : workspace of infv2_select_blocks_workspace(prob, S_cmp != NULL)
 *           bytes; its contents need no initialisation and are not kept
 *           between calls.  Calls that share a workspace must not overlap. */
size_t infv2_select_blocks_workspace(const infv2_problem* prob, int with_scores);
int infv2_select_blocks(const infv2_problem* prob, const void* Q, const void* Kc1,
                        const void* Kc2, float* S_cmp, int32_t* idx, int32_t* n_sel,
                        void* ws, size_t ws_bytes, void* stream);

/* The decode step's K^C1 append and the block selection in one call:
 * kernels [c1_begin, c1_end) of every sequence are formed from K exactly as
 * infv2_compress_k forms them (papernotes note, 关键设计 3: the mean of the
 * kernel's keys, rounded once) and written to Kc1, and the selection runs as
 * infv2_select_blocks with S_cmp = NULL and no K^C2; the appended kernels are
 * formed inside the score sweep that reads them, so the step needs no
 * separate compress launch (OpenBMB blog, 查询和键值词元的不同粒度: token-level
 * queries make decode sparse, so the per-step work is what matters).  Kc1,
 * idx and n_sel are bitwise those of infv2_compress_k(c1_begin, c1_end)
 * followed by infv2_select_blocks.
 *   K     : [batch][kv_cap][h_kv][d] (input)
 *   Kc1   : [batch][h_kv][c1_cap][d] (input; rows [c1_begin, c1_end) are
 *           written and are not read)
 *   c1_begin, c1_end : 0 <= c1_begin <= c1_end <= n_C1 (else INFV2_E_ARG)
 *   idx, n_sel, ws, ws_bytes : as in infv2_select_blocks (workspace of
 *           infv2_select_blocks_workspace(prob, 0) bytes)
 * Serves the decode shapes of infv2_select_blocks (bf16, G = 16, d = 128,
 * n_q <= 4, k <= 32) with the exact LSE; anything else is refused with
 * INFV2_E_UNSUPPORTED before any work is enqueued. */
int infv2_select_blocks_append(const infv2_problem* prob, const void* Q, const void* K,
                               void* Kc1, int32_t c1_begin, int32_t c1_end, int32_t* idx,
                               int32_t* n_sel, void* ws, size_t ws_bytes, void* stream);

/* Block-sparse attention (paperlayer.ai summary, A IMPLEMENTATION DETAIL):
 * for each query token and head, softmax attention over the keys
 * T(p) = {t <= p : floor(t/B) in I(p)}, returning O and the natural-log LSE.
 *   Q     : [batch][n_q][h_q][d]        K, V : [batch][kv_cap][h_kv][d]
 *   idx, n_sel : as written by infv2_topk_select (any ascending sets of
 *           distinct causal blocks whose last entry is b_p are accepted)
 *   O     : [batch][n_q][h_q][d] I/O dtype (output, rounded once)
 *   lse   : [batch][h_q][n_q] fp32 (output; may be NULL)
 *   ws    : workspace of infv2_sparse_attn_workspace(prob) bytes. */
size_t infv2_sparse_attn_workspace(const infv2_problem* prob);
int infv2_sparse_attn(const infv2_problem* prob, const void* Q, const void* K,
                      const void* V, const int32_t* idx, const int32_t* n_sel,
                      void* O, float* lse, void* ws, size_t ws_bytes, void* stream);

/* The whole decode step in one call (OpenBMB blog, 查询和键值词元的不同粒度:
 * with token-level queries the per-step selection and attention are the
 * decode cost): infv2_select_blocks_append followed by infv2_sparse_attn,
 * with the selection's last stage -- merging the per-chunk candidate lists
 * into I(p) -- done by the attention's split workgroups themselves, so the
 * step has one launch fewer.  Kc1, idx, n_sel, O and lse are bitwise those of
 * the two calls.
 *   Q, K, V, Kc1, c1_begin, c1_end : as in infv2_select_blocks_append (V as
 *           in infv2_sparse_attn)
 *   idx, n_sel : [batch][h_kv][n_q][budget], [batch][h_kv][n_q] (output)
 *   O, lse : as in infv2_sparse_attn (output; lse may be NULL)
 *   ws    : workspace of infv2_decode_step_workspace(prob) bytes.
 * Serves the decode shapes of both calls (bf16, G = 16, d = 128, B = 64,
 * n_q <= 4, k <= 32, exact LSE, one length for all sequences); anything else
 * is refused with INFV2_E_UNSUPPORTED before any work is enqueued. */
size_t infv2_decode_step_workspace(const infv2_problem* prob);
int infv2_decode_step(const infv2_problem* prob, const void* Q, const void* K, const void* V,
                      void* Kc1, int32_t c1_begin, int32_t c1_end, int32_t* idx,
                      int32_t* n_sel, void* O, float* lse, void* ws, size_t ws_bytes,
                      void* stream);

/* Dense causal attention, the dense branch of the dense-sparse switch
 * (papernotes.org InfLLM-V2 note, 方法详解 > 整体框架 flowchart: short inputs take
 * ordinary dense attention; OpenBMB blog "技术Blog-4 | 新一代InfLLM：可训练的稀疏
 * 注意力机制", 动态上下文块选择 > 语义核: when the sequence fits in the selected
 * blocks the sparse attention degenerates to dense), and the baseline it is
 * timed against.  The same as infv2_sparse_attn with T(p) = {0..p}: every
 * causal key.  Layouts, ownership and errors as above;
 * ws: workspace of infv2_dense_attn_workspace(prob) bytes. */
size_t infv2_dense_attn_workspace(const infv2_problem* prob);
int infv2_dense_attn(const infv2_problem* prob, const void* Q, const void* K,
                     const void* V, void* O, float* lse, void* ws, size_t ws_bytes,
                     void* stream);

/* Backward of the block-sparse attention for training (OpenBMB blog,
 * 可训练稀疏注意力的设计原则: the top-k selection is not differentiable and the
 * kernels are parameter-free means trained through the token keys, so the
 * gradients are those of the attention with the sets I(p) held fixed).  Per
 * query token and head, over T(p) = {t <= p : floor(t/B) in I(p)}:
 *   P_t = exp(scale q.k_t - lse),  dP_t = dO.v_t,  D = dO.O,
 *   dZ_t = P_t (dP_t - D),  dQ = scale sum_t dZ_t k_t,
 *   dK_t += scale dZ_t q,  dV_t += P_t dO  (summed over the query tokens).
 *   Q, K, V, idx, n_sel : as given to infv2_sparse_attn
 *   O, lse : its outputs (lse required)
 *   dO    : [batch][n_q][h_q][d] I/O dtype, the gradient of O
 *   dQ    : [batch][n_q][h_q][d] fp32 (output)
 *   dK, dV: [batch][kv_cap][h_kv][d] fp32 (output; rows 0..n_kv-1 are
 *           written, zero where no query attends)
 *   ws    : workspace of infv2_sparse_attn_bwd_workspace(prob) bytes.
 * dQ is deterministic; the bf16 kernels add the partial dK / dV of different
 * query windows with atomics, so their last bits may differ between runs. */
size_t infv2_sparse_attn_bwd_workspace(const infv2_problem* prob);
int infv2_sparse_attn_bwd(const infv2_problem* prob, const void* Q, const void* K,
                          const void* V, const int32_t* idx, const int32_t* n_sel,
                          const void* O, const float* lse, const void* dO, float* dQ,
                          float* dK, float* dV, void* ws, size_t ws_bytes, void* stream);

/* The same for dense causal attention (T(p) = {0..p}), the backward of
 * infv2_dense_attn; ws: infv2_dense_attn_bwd_workspace(prob) bytes. */
size_t infv2_dense_attn_bwd_workspace(const infv2_problem* prob);
int infv2_dense_attn_bwd(const infv2_problem* prob, const void* Q, const void* K,
                         const void* V, const void* O, const float* lse, const void* dO,
                         float* dQ, float* dK, float* dV, void* ws, size_t ws_bytes,
                         void* stream);

/* Varlen batches and a paged K/V cache, for serving decode (OpenBMB blog,
 * 查询和键值词元的不同粒度: token-level queries are what makes the sparse
 * decode step fast; the paged layout is this library's own serving format).
 * The definitions are those of the calls above, applied to each sequence
 * with its own length:
 *  - seq_lens : [batch] int32 (device): sequence i's cache holds seq_lens[i]
 *    tokens, the new ones included; its n_q query tokens are its last n_q,
 *    at positions seq_lens[i]-n_q .. seq_lens[i]-1.  Entries must lie in
 *    [n_q, n_kv]; values outside are clamped into that range on the device.
 *    prob->n_kv is the longest length any sequence may have (it sizes the
 *    grids and workspaces); prob->q_pos0 is not used (pass 0).
 *  - Paged cache: K and V are pools of n_pages pages [B][h_kv][d] (bf16);
 *    block_table [batch][max_blocks] int32 (device) gives the page of block j
 *    of sequence i, for j < ceil(seq_lens[i]/B) (max_blocks >= ceil(n_kv/B)).
 *    A page holds one KV block, so a selected block is read from one page.
 *    Entries outside [0, n_pages) are clamped into it (that sequence's
 *    result is then meaningless, but nothing is read out of the pool).
 *    block_table == NULL: contiguous K, V [batch][kv_cap][h_kv][d].
 *  - K^C1 (and K^C2) stay contiguous per sequence, [batch][h_kv][c1_cap][d].
 * Decode shapes only: bf16, G = 16, d = 128, B = 64, l_C1 = 32, s_C1 = 16,
 * n_q <= 4, k <= 32, budget <= 64 (others: INFV2_E_UNSUPPORTED).
 *
 * infv2_compress_k_varlen: stage 1 (coarse = 0: K^C1 into Kc [batch][h_kv]
 * [c1_cap][d]) or the coarse keys of the LSE approximation (coarse = 1: K^C2
 * into [batch][h_kv][c2_cap][d]) for each sequence's last `last_n` complete
 * kernels (all of them when last_n <= 0), with the definitions of
 * infv2_compress_k / infv2_compress_k2.  A decode step passes last_n = 1
 * (rewriting a kernel that exists already is harmless). */
int infv2_compress_k_varlen(const infv2_problem* prob, const void* K,
                            const int32_t* block_table, int32_t max_blocks, int32_t n_pages,
                            const int32_t* seq_lens, void* Kc, int32_t coarse,
                            int32_t last_n, void* stream);

/* infv2_select_blocks for a varlen batch: idx [batch][h_kv][n_q][budget],
 * n_sel [batch][h_kv][n_q] as in infv2_topk_select, each row with its own
 * sequence's positions and kernels (S^cmp is not produced).  Kc2 with
 * prob->lse_approx.  ws: infv2_select_blocks_varlen_workspace(prob) bytes,
 * not kept between calls. */
size_t infv2_select_blocks_varlen_workspace(const infv2_problem* prob);
int infv2_select_blocks_varlen(const infv2_problem* prob, const void* Q, const void* Kc1,
                               const void* Kc2, const int32_t* seq_lens, int32_t* idx,
                               int32_t* n_sel, void* ws, size_t ws_bytes, void* stream);

/* infv2_sparse_attn for a varlen batch, from a paged (block_table set) or
 * contiguous cache: O [batch][n_q][h_q][d], lse [batch][h_q][n_q] (may be
 * NULL).  ws: infv2_sparse_attn_varlen_workspace(prob) bytes. */
size_t infv2_sparse_attn_varlen_workspace(const infv2_problem* prob);
int infv2_sparse_attn_varlen(const infv2_problem* prob, const void* Q, const void* K,
                             const void* V, const int32_t* block_table, int32_t max_blocks,
                             int32_t n_pages, const int32_t* seq_lens, const int32_t* idx,
                             const int32_t* n_sel, void* O, float* lse, void* ws,
                             size_t ws_bytes, void* stream);

const char* infv2_status_string(int status);
const char* infv2_last_error(void);

/* infv2_sparse_attn for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation, kernels and outputs, bit for bit, but
 * its workspace is a static device array of INFV2_NOALLOC_SCRATCH_BYTES
 * inside the library (one copy per GPU, held until the process ends) instead
 * of a caller buffer.  It calls no hipMalloc / hipFree and nothing that
 * allocates.  The caller still passes every input and output, as for
 * infv2_sparse_attn.
 *  - A problem whose infv2_sparse_attn_workspace(prob) exceeds the scratch
 *    is refused with INFV2_E_WORKSPACE before anything is enqueued.
 *  - The scratch's address is looked up once per GPU, on the first call
 *    with that GPU current; `stream` must belong to the current GPU
 *    (INFV2_E_ARG otherwise), and a failed lookup returns INFV2_E_HIP.
 *  - All calls on one GPU share its scratch and no call clears it (the
 *    kernels write every byte they read).  Calls that can overlap on one
 *    GPU (other streams, other threads) race on it: serialise them. */
#define INFV2_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int infv2_sparse_attn_noalloc(const infv2_problem* prob, const void* Q, const void* K,
                              const void* V, const int32_t* idx, const int32_t* n_sel,
                              void* O, float* lse, void* stream);

/* Identity of this build: the first 16 hex digits of the SHA-256 of the
 * library's source files (csrc/ and this header), fixed when the library was
 * compiled.  A caller compares it with the sources it holds to know that the
 * loaded library was built from them.  Static string, never NULL. */
const char* infv2_build_id(void);

#ifdef __cplusplus
}
#endif
#endif /* INFV2_H */
