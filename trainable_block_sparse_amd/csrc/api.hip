// Host side of the C ABI declared in include/infv2.h: argument validation,
// workspace sizing and kernel dispatch.  No allocation, no synchronisation.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>

#include "common.hpp"
#include "select_merge.hpp"

namespace infv2 {
hipError_t launch_compress_k(const infv2_problem& p, const void* K, void* Kc1, int c1_begin,
                             int c1_end, int64_t kv_cap, int64_t c1_cap, int l_len, int s_len,
                             hipStream_t stream);
hipError_t launch_compress_k_varlen(const infv2_problem& p, const void* K,
                                    const int32_t* block_table, int max_blocks, int n_pages,
                                    const int32_t* seq_lens, void* Kc, int64_t kv_cap,
                                    int64_t c_cap, int l_len, int s_len, int last_n,
                                    hipStream_t stream);
hipError_t launch_select_varlen(const infv2_problem& p, const void* Q, const KeySet& ks,
                                const int32_t* seq_lens, int32_t* idx, int32_t* n_sel, void* ws,
                                int n_blk, float scale, int budget, hipStream_t stream);
hipError_t launch_attn_varlen(const infv2_problem& p, const void* Q, const void* K,
                              const void* V, const int32_t* block_table, int max_blocks,
                              int n_pages, const int32_t* seq_lens, const int32_t* idx,
                              const int32_t* n_sel, void* O, float* lse, void* ws, int budget,
                              int64_t kv_cap, float scale, hipStream_t stream);
bool scores_use_split(const infv2_problem& p);
bool attn_use_split(const infv2_problem& p);
bool scores_fast_shape(const infv2_problem& p);
size_t scores_workspace(const infv2_problem& p, const KeySet& ks);
size_t scores_generic_lds(const infv2_problem& p, int n_c1);
hipError_t launch_block_scores(const infv2_problem& p, const void* Q, const KeySet& ks,
                               float* S_cmp, float* S_sh, void* ws, int n_blk, float scale,
                               hipStream_t stream);
hipError_t launch_topk(const infv2_problem& p, const float* S_cmp, int32_t* idx, int32_t* n_sel,
                       int n_blk, int budget, hipStream_t stream);
bool select_fused_shape(const infv2_problem& p, int n_c1);
size_t select_fused_workspace(const infv2_problem& p, int n_c1);
hipError_t launch_select_fused(const infv2_problem& p, const void* Q, const KeySet& ks,
                               float* S_cmp, int32_t* idx, int32_t* n_sel, void* ws, int n_blk,
                               float scale, int budget, hipStream_t stream);
hipError_t launch_select_append(const infv2_problem& p, const void* Q, const void* K, void* Kc1,
                                int c1_begin, int c1_end, int64_t kv_cap, const KeySet& ks,
                                int32_t* idx, int32_t* n_sel, void* ws, int n_blk, float scale,
                                int budget, hipStream_t stream, CandLists* lists = nullptr);
hipError_t launch_attn_decode_select(const infv2_problem& p, const void* Q, const void* K,
                                     const void* V, const CandLists& lists, int32_t* idx,
                                     int32_t* n_sel, void* O, float* lse, void* ws, int budget,
                                     int64_t kv_cap, float scale, hipStream_t stream);
bool attn_fast_shape(const infv2_problem& p);
size_t attn_workspace(const infv2_problem& p, int budget, bool sparse);
hipError_t launch_attn(const infv2_problem& p, const void* Q, const void* K, const void* V,
                       const int32_t* idx, const int32_t* n_sel, void* O, float* lse, void* ws,
                       int budget, int64_t kv_cap, float scale, hipStream_t stream);
size_t attn_bwd_workspace(const infv2_problem& p, bool sparse);
size_t attn_bwd_generic_lds(const infv2_problem& p, int budget, bool sparse);
hipError_t launch_attn_bwd(const infv2_problem& p, const void* Q, const void* K, const void* V,
                           const int32_t* idx, const int32_t* n_sel, const void* O,
                           const float* lse, const void* dO, float* dQ, float* dK, float* dV,
                           void* ws, int budget, int64_t kv_cap, float scale,
                           hipStream_t stream);
}  // namespace infv2

using namespace infv2;

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int ok() {
  g_last_error.clear();
  return INFV2_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(INFV2_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }
bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; }

// The size helpers return 0 for a problem whose strides are not positive
// (check() rejects such a problem; the helpers only must not divide by zero).
int n_c1_of(const infv2_problem& p) {
  if (p.s_C1 <= 0 || p.l_C1 <= 0) return 0;
  return p.n_kv < p.l_C1 ? 0 : (p.n_kv - p.l_C1) / p.s_C1 + 1;
}
// coarse kernels of the LSE approximation: l_C2 = 4 l_C1, s_C2 = 4 s_C1
int l_c2_of(const infv2_problem& p) { return 4 * p.l_C1; }
int s_c2_of(const infv2_problem& p) { return 4 * p.s_C1; }
int n_c2_of(const infv2_problem& p) {
  if (p.s_C1 <= 0 || p.l_C1 <= 0) return 0;
  return p.n_kv < l_c2_of(p) ? 0 : (p.n_kv - l_c2_of(p)) / s_c2_of(p) + 1;
}
int n_blk_of(const infv2_problem& p) { return p.B <= 0 ? 0 : (p.n_kv + p.B - 1) / p.B; }
int budget_of(const infv2_problem& p) { return p.N_init + p.N_local + p.k; }
int64_t kv_cap_of(const infv2_problem& p) { return p.kv_cap ? p.kv_cap : p.n_kv; }
int64_t c1_cap_of(const infv2_problem& p) { return p.c1_cap ? p.c1_cap : n_c1_of(p); }
int64_t c2_cap_of(const infv2_problem& p) { return p.c2_cap ? p.c2_cap : n_c2_of(p); }
KeySet keys_of(const infv2_problem& p, const void* Kc1, const void* Kc2) {
  KeySet ks;
  ks.Kc1 = Kc1;
  ks.Kc2 = p.lse_approx ? Kc2 : nullptr;
  ks.n_c1 = n_c1_of(p);
  ks.n_c2 = n_c2_of(p);
  ks.c1_cap = c1_cap_of(p);
  ks.c2_cap = c2_cap_of(p);
  return ks;
}
float scale_of(const infv2_problem& p) {
  return p.scale != 0.0f ? p.scale : 1.0f / sqrtf((float)p.d);
}

// Shape and parameter checks shared by every entry point.
int check(const infv2_problem* pp) {
  if (!pp) return fail(INFV2_E_ARG, "prob is NULL");
  const infv2_problem& p = *pp;
  if (p.batch < 1 || p.n_q < 1 || p.n_kv < 1 || p.h_kv < 1 || p.G < 1 || p.d < 1)
    return fail(INFV2_E_ARG, "batch, n_q, n_kv, h_kv, G and d must be >= 1");
  if (p.q_pos0 < 0 || (int64_t)p.q_pos0 + p.n_q > p.n_kv)
    return fail(INFV2_E_ARG, "need 0 <= q_pos0 and q_pos0 + n_q <= n_kv (got %d + %d > %d)",
                p.q_pos0, p.n_q, p.n_kv);
  if (p.dtype != INFV2_BF16 && p.dtype != INFV2_F32)
    return fail(INFV2_E_ARG, "dtype must be INFV2_BF16 or INFV2_F32");
  if (p.B < 1 || p.l_C1 < 1 || p.s_C1 < 1 || p.k < 0 || p.N_init < 0 || p.N_local < 1)
    return fail(INFV2_E_ARG, "need B, l_C1, s_C1, N_local >= 1 and k, N_init >= 0");
  if (p.B % p.s_C1 != 0)
    return fail(INFV2_E_ARG, "B (%d) must be a multiple of s_C1 (%d)", p.B, p.s_C1);
  // stage-3 parameters must be the stride and count of the kernels that
  // intersect one block: s = B/s_C1, l = B/s_C1 + floor((l_C1-1)/s_C1)
  const int s_expect = p.B / p.s_C1;
  const int l_expect = s_expect + (p.l_C1 - 1) / p.s_C1;
  if (p.s != s_expect || p.l != l_expect)
    return fail(INFV2_E_ARG,
                "max-pool (l=%d, s=%d) must equal the count and stride of the kernels "
                "intersecting a block (l=%d, s=%d)",
                p.l, p.s, l_expect, s_expect);
  if (!(p.scale >= 0.0f) || isinf(p.scale))
    return fail(INFV2_E_ARG, "scale must be finite and >= 0 (0 selects 1/sqrt(d))");
  if (p.kv_cap != 0 && p.kv_cap < p.n_kv)
    return fail(INFV2_E_ARG, "kv_cap (%lld) < n_kv (%d)", (long long)p.kv_cap, p.n_kv);
  if (p.c1_cap != 0 && p.c1_cap < n_c1_of(p))
    return fail(INFV2_E_ARG, "c1_cap (%lld) < n_C1 (%d)", (long long)p.c1_cap, n_c1_of(p));
  if (p.c2_cap != 0 && p.c2_cap < n_c2_of(p))
    return fail(INFV2_E_ARG, "c2_cap (%lld) < n_C2 (%d)", (long long)p.c2_cap, n_c2_of(p));
  if (p.lse_approx != 0 && p.lse_approx != 1) return fail(INFV2_E_ARG, "lse_approx must be 0 or 1");
  if (budget_of(p) < 1) return fail(INFV2_E_ARG, "N_init + N_local + k must be >= 1");
  if ((int64_t)p.G * p.h_kv > 4096) return fail(INFV2_E_ARG, "h_q too large");
  // launch grids carry the batch (times up to 4 query tokens on the decode
  // paths) in a dimension of at most 65535 workgroups
  if ((int64_t)p.batch * std::min(p.n_q, 4) > 65535)
    return fail(INFV2_E_UNSUPPORTED, "batch (%d) x min(n_q, 4) exceeds 65535: split the batch",
                p.batch);
  // kernel instances
  if (!is_pow2(p.l_C1))
    return fail(INFV2_E_UNSUPPORTED, "l_C1 (%d) must be a power of two (exact mean)", p.l_C1);
  if (p.d > 256 || p.d % 8 != 0)
    return fail(INFV2_E_UNSUPPORTED, "d (%d) must be a multiple of 8 and <= 256", p.d);
  if (p.dtype == INFV2_BF16 && p.d % 8 != 0)
    return fail(INFV2_E_UNSUPPORTED, "bf16 rows must be 16-byte multiples");
  if (!scores_fast_shape(p) && scores_generic_lds(p, n_c1_of(p)) > 60 * 1024)
    return fail(INFV2_E_UNSUPPORTED,
                "n_C1 = %d too large for the generic selection kernel (shape G=%d d=%d dtype=%d)",
                n_c1_of(p), p.G, p.d, p.dtype);
  return INFV2_OK;
}

#define CHECK_PTR(ptr)                                                          \
  do {                                                                          \
    if (!(ptr)) return fail(INFV2_E_ARG, "%s is NULL", #ptr);                   \
    if (!aligned16(ptr)) return fail(INFV2_E_ARG, "%s is not 16-byte aligned", #ptr); \
  } while (0)

}  // namespace

extern "C" {

int32_t infv2_n_kernels(const infv2_problem* p) { return p ? n_c1_of(*p) : -1; }
int32_t infv2_n_coarse_kernels(const infv2_problem* p) { return p ? n_c2_of(*p) : -1; }
int32_t infv2_n_blocks(const infv2_problem* p) { return p ? n_blk_of(*p) : -1; }
int32_t infv2_budget(const infv2_problem* p) { return p ? budget_of(*p) : -1; }

int infv2_use_dense(const infv2_problem* p) {
  if (check(p) != INFV2_OK) return -1;
  return n_blk_of(*p) <= budget_of(*p) ? 1 : 0;
}

int infv2_check_problem(const infv2_problem* p) {
  const int st = check(p);
  return st == INFV2_OK ? ok() : st;
}

int infv2_compress_k(const infv2_problem* p, const void* K, void* Kc1, int32_t c1_begin,
                     int32_t c1_end, void* stream) {
  int st = check(p);
  if (st) return st;
  CHECK_PTR(K);
  CHECK_PTR(Kc1);
  const int n_c1 = n_c1_of(*p);
  if (c1_begin < 0 || c1_begin > c1_end || c1_end > n_c1)
    return fail(INFV2_E_ARG, "need 0 <= c1_begin <= c1_end <= n_C1 (%d..%d, n_C1=%d)",
                c1_begin, c1_end, n_c1);
  return hip_status(launch_compress_k(*p, K, Kc1, c1_begin, c1_end, kv_cap_of(*p), c1_cap_of(*p),
                                      p->l_C1, p->s_C1, (hipStream_t)stream),
                    "infv2_compress_k");
}

int infv2_compress_k2(const infv2_problem* p, const void* K, void* Kc2, int32_t c2_begin,
                      int32_t c2_end, void* stream) {
  int st = check(p);
  if (st) return st;
  CHECK_PTR(K);
  CHECK_PTR(Kc2);
  const int n_c2 = n_c2_of(*p);
  if (c2_begin < 0 || c2_begin > c2_end || c2_end > n_c2)
    return fail(INFV2_E_ARG, "need 0 <= c2_begin <= c2_end <= n_C2 (%d..%d, n_C2=%d)",
                c2_begin, c2_end, n_c2);
  return hip_status(launch_compress_k(*p, K, Kc2, c2_begin, c2_end, kv_cap_of(*p), c2_cap_of(*p),
                                      l_c2_of(*p), s_c2_of(*p), (hipStream_t)stream),
                    "infv2_compress_k2");
}

size_t infv2_block_scores_workspace(const infv2_problem* p) {
  if (check(p) != INFV2_OK) return 0;
  return scores_workspace(*p, keys_of(*p, nullptr, nullptr));
}

// The key pointers a selection call needs: K^C1 when a kernel exists, K^C2
// with the LSE approximation when a coarse kernel exists.
static int check_keys(const infv2_problem& p, const void* Kc1, const void* Kc2) {
  if (n_c1_of(p) > 0) CHECK_PTR(Kc1);
  if (p.lse_approx && n_c2_of(p) > 0) CHECK_PTR(Kc2);
  return INFV2_OK;
}

int infv2_block_scores(const infv2_problem* p, const void* Q, const void* Kc1, const void* Kc2,
                       float* S_cmp, float* S_shared, void* ws, size_t ws_bytes, void* stream) {
  int st = check(p);
  if (st) return st;
  CHECK_PTR(Q);
  CHECK_PTR(S_cmp);
  if (S_shared && !aligned16(S_shared))
    return fail(INFV2_E_ARG, "S_shared is not 16-byte aligned");
  if ((st = check_keys(*p, Kc1, Kc2))) return st;
  const KeySet ks = keys_of(*p, Kc1, Kc2);
  const size_t need = scores_workspace(*p, ks);
  if (need) {
    CHECK_PTR(ws);
    if (ws_bytes < need)
      return fail(INFV2_E_WORKSPACE, "block_scores workspace %zu < %zu bytes", ws_bytes, need);
  }
  return hip_status(launch_block_scores(*p, Q, ks, S_cmp, S_shared, ws, n_blk_of(*p),
                                        scale_of(*p), (hipStream_t)stream),
                    "infv2_block_scores");
}

int infv2_topk_select(const infv2_problem* p, const float* S_cmp, int32_t* idx, int32_t* n_sel,
                      void* stream) {
  int st = check(p);
  if (st) return st;
  CHECK_PTR(S_cmp);
  CHECK_PTR(idx);
  CHECK_PTR(n_sel);
  return hip_status(
      launch_topk(*p, S_cmp, idx, n_sel, n_blk_of(*p), budget_of(*p), (hipStream_t)stream),
      "infv2_topk_select");
}

size_t infv2_select_blocks_workspace(const infv2_problem* p, int with_scores) {
  if (check(p) != INFV2_OK) return 0;
  const KeySet ks = keys_of(*p, nullptr, nullptr);
  const size_t base = scores_workspace(*p, ks);
  if (select_fused_shape(*p, ks.n_c1)) return align256(base) + select_fused_workspace(*p, ks.n_c1);
  if (with_scores) return base;
  const size_t rows = (size_t)p->batch * p->n_q * p->h_kv;
  return align256(base) + rows * (size_t)n_blk_of(*p) * sizeof(float);
}

int infv2_select_blocks(const infv2_problem* p, const void* Q, const void* Kc1, const void* Kc2,
                        float* S_cmp, int32_t* idx, int32_t* n_sel, void* ws, size_t ws_bytes,
                        void* stream) {
  int st = check(p);
  if (st) return st;
  CHECK_PTR(Q);
  CHECK_PTR(idx);
  CHECK_PTR(n_sel);
  if (S_cmp && !aligned16(S_cmp)) return fail(INFV2_E_ARG, "S_cmp is not 16-byte aligned");
  if ((st = check_keys(*p, Kc1, Kc2))) return st;
  const KeySet ks = keys_of(*p, Kc1, Kc2);
  const size_t need = infv2_select_blocks_workspace(p, S_cmp != nullptr);
  if (need) {
    CHECK_PTR(ws);
    if (ws_bytes < need)
      return fail(INFV2_E_WORKSPACE, "select_blocks workspace %zu < %zu bytes", ws_bytes, need);
  }
  const hipStream_t s = (hipStream_t)stream;
  if (select_fused_shape(*p, ks.n_c1)) {
    return hip_status(launch_select_fused(*p, Q, ks, S_cmp, idx, n_sel, ws, n_blk_of(*p),
                                          scale_of(*p), budget_of(*p), s),
                      "infv2_select_blocks");
  }
  float* S = S_cmp ? S_cmp : (float*)((char*)ws + align256(scores_workspace(*p, ks)));
  hipError_t e = launch_block_scores(*p, Q, ks, S, nullptr, ws, n_blk_of(*p), scale_of(*p), s);
  if (e == hipSuccess) e = launch_topk(*p, S, idx, n_sel, n_blk_of(*p), budget_of(*p), s);
  return hip_status(e, "infv2_select_blocks");
}

int infv2_select_blocks_append(const infv2_problem* p, const void* Q, const void* K, void* Kc1,
                               int32_t c1_begin, int32_t c1_end, int32_t* idx, int32_t* n_sel,
                               void* ws, size_t ws_bytes, void* stream) {
  int st = check(p);
  if (st) return st;
  CHECK_PTR(Q);
  CHECK_PTR(K);
  CHECK_PTR(idx);
  CHECK_PTR(n_sel);
  if (p->lse_approx || !scores_use_split(*p) || !select_fused_shape(*p, n_c1_of(*p)))
    return fail(INFV2_E_UNSUPPORTED,
                "select_blocks_append serves the decode shapes of infv2_select_blocks (bf16, "
                "G=16, d=128, n_q<=4, k<=32, exact LSE)");
  if ((st = check_keys(*p, Kc1, nullptr))) return st;
  const KeySet ks = keys_of(*p, Kc1, nullptr);
  if (c1_begin < 0 || c1_begin > c1_end || c1_end > ks.n_c1)
    return fail(INFV2_E_ARG, "need 0 <= c1_begin <= c1_end <= n_C1 (%d..%d, n_C1=%d)",
                c1_begin, c1_end, ks.n_c1);
  const size_t need = infv2_select_blocks_workspace(p, 0);
  if (need) {
    CHECK_PTR(ws);
    if (ws_bytes < need)
      return fail(INFV2_E_WORKSPACE, "select_blocks_append workspace %zu < %zu bytes", ws_bytes,
                  need);
  }
  return hip_status(launch_select_append(*p, Q, K, Kc1, c1_begin, c1_end, kv_cap_of(*p), ks, idx,
                                         n_sel, ws, n_blk_of(*p), scale_of(*p), budget_of(*p),
                                         (hipStream_t)stream),
                    "infv2_select_blocks_append");
}

size_t infv2_decode_step_workspace(const infv2_problem* p) {
  if (check(p) != INFV2_OK) return 0;
  return align256(infv2_select_blocks_workspace(p, 0)) + attn_workspace(*p, budget_of(*p), true);
}

int infv2_decode_step(const infv2_problem* p, const void* Q, const void* K, const void* V,
                      void* Kc1, int32_t c1_begin, int32_t c1_end, int32_t* idx, int32_t* n_sel,
                      void* O, float* lse, void* ws, size_t ws_bytes, void* stream) {
  int st = check(p);
  if (st) return st;
  CHECK_PTR(Q);
  CHECK_PTR(K);
  CHECK_PTR(V);
  CHECK_PTR(idx);
  CHECK_PTR(n_sel);
  CHECK_PTR(O);
  CHECK_PTR(ws);
  if (lse && !aligned16(lse)) return fail(INFV2_E_ARG, "lse is not 16-byte aligned");
  if (p->lse_approx || !scores_use_split(*p) || !attn_use_split(*p) ||
      !select_fused_shape(*p, n_c1_of(*p)))
    return fail(INFV2_E_UNSUPPORTED,
                "decode_step serves the decode shapes of infv2_select_blocks_append and "
                "infv2_sparse_attn (bf16, G=16, d=128, B=64, n_q<=4, k<=32, exact LSE)");
  if ((st = check_keys(*p, Kc1, nullptr))) return st;
  const KeySet ks = keys_of(*p, Kc1, nullptr);
  if (c1_begin < 0 || c1_begin > c1_end || c1_end > ks.n_c1)
    return fail(INFV2_E_ARG, "need 0 <= c1_begin <= c1_end <= n_C1 (%d..%d, n_C1=%d)",
                c1_begin, c1_end, ks.n_c1);
  const size_t need = infv2_decode_step_workspace(p);
  if (ws_bytes < need)
    return fail(INFV2_E_WORKSPACE, "decode_step workspace %zu < %zu bytes", ws_bytes, need);
  const hipStream_t s = (hipStream_t)stream;
  CandLists lists{};
  hipError_t e = launch_select_append(*p, Q, K, Kc1, c1_begin, c1_end, kv_cap_of(*p), ks, idx,
                                      n_sel, ws, n_blk_of(*p), scale_of(*p), budget_of(*p), s,
                                      &lists);
  if (e == hipSuccess)
    e = launch_attn_decode_select(*p, Q, K, V, lists, idx, n_sel, O, lse,
                                  (char*)ws + align256(infv2_select_blocks_workspace(p, 0)),
                                  budget_of(*p), kv_cap_of(*p), scale_of(*p), s);
  return hip_status(e, "infv2_decode_step");
}

size_t infv2_sparse_attn_workspace(const infv2_problem* p) {
  if (check(p) != INFV2_OK) return 0;
  return attn_workspace(*p, budget_of(*p), true);
}

int infv2_sparse_attn(const infv2_problem* p, const void* Q, const void* K, const void* V,
                      const int32_t* idx, const int32_t* n_sel, void* O, float* lse, void* ws,
                      size_t ws_bytes, void* stream) {
  int st = check(p);
  if (st) return st;
  CHECK_PTR(Q);
  CHECK_PTR(K);
  CHECK_PTR(V);
  CHECK_PTR(idx);
  CHECK_PTR(n_sel);
  CHECK_PTR(O);
  if (lse && !aligned16(lse)) return fail(INFV2_E_ARG, "lse is not 16-byte aligned");
  const size_t need = attn_workspace(*p, budget_of(*p), true);
  if (need) {
    CHECK_PTR(ws);
    if (ws_bytes < need)
      return fail(INFV2_E_WORKSPACE, "sparse_attn workspace %zu < %zu bytes", ws_bytes, need);
  }
  return hip_status(launch_attn(*p, Q, K, V, idx, n_sel, O, lse, ws, budget_of(*p), kv_cap_of(*p),
                                scale_of(*p), (hipStream_t)stream),
                    "infv2_sparse_attn");
}

// Workspace of infv2_sparse_attn_noalloc: one copy on every GPU the library
// runs on.  Host code never uses this name as an address: the per-device
// address from hipGetSymbolAddress is what kernels receive.
static __device__ __align__(256) unsigned char scratch[INFV2_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch`, per device

// Address of this GPU's scratch; looked up once per device, with the device
// current.  The stream must belong to the current device.
int scratch_of(hipStream_t stream, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(INFV2_E_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(INFV2_E_UNSUPPORTED, "device %d is past the %d the scratch table holds", dev,
                kMaxDevices);
  if (stream != nullptr) {
    int sdev = -1;
    e = hipStreamGetDevice(stream, &sdev);
    if (e != hipSuccess) return fail(INFV2_E_HIP, "hipStreamGetDevice: %s", hipGetErrorString(e));
    if (sdev != dev)
      return fail(INFV2_E_ARG, "stream belongs to device %d but device %d is current", sdev, dev);
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr)
      return fail(INFV2_E_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return INFV2_OK;
}
}  // namespace

int infv2_sparse_attn_noalloc(const infv2_problem* p, const void* Q, const void* K,
                              const void* V, const int32_t* idx, const int32_t* n_sel, void* O,
                              float* lse, void* stream) {
  int st = check(p);
  if (st) return st;
  CHECK_PTR(Q);
  CHECK_PTR(K);
  CHECK_PTR(V);
  CHECK_PTR(idx);
  CHECK_PTR(n_sel);
  CHECK_PTR(O);
  if (lse && !aligned16(lse)) return fail(INFV2_E_ARG, "lse is not 16-byte aligned");
  const size_t need = attn_workspace(*p, budget_of(*p), true);
  if (need > INFV2_NOALLOC_SCRATCH_BYTES)
    return fail(INFV2_E_WORKSPACE,
                "sparse_attn_noalloc: this problem needs %zu bytes of workspace, more than the "
                "%zu-byte static scratch",
                need, (size_t)INFV2_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if (need && (st = scratch_of((hipStream_t)stream, &ws))) return st;
  return hip_status(launch_attn(*p, Q, K, V, idx, n_sel, O, lse, ws, budget_of(*p), kv_cap_of(*p),
                                scale_of(*p), (hipStream_t)stream),
                    "infv2_sparse_attn_noalloc");
}

size_t infv2_dense_attn_workspace(const infv2_problem* p) {
  if (check(p) != INFV2_OK) return 0;
  return attn_workspace(*p, budget_of(*p), false);
}

int infv2_dense_attn(const infv2_problem* p, const void* Q, const void* K, const void* V,
                     void* O, float* lse, void* ws, size_t ws_bytes, void* stream) {
  int st = check(p);
  if (st) return st;
  CHECK_PTR(Q);
  CHECK_PTR(K);
  CHECK_PTR(V);
  CHECK_PTR(O);
  if (lse && !aligned16(lse)) return fail(INFV2_E_ARG, "lse is not 16-byte aligned");
  const size_t need = attn_workspace(*p, budget_of(*p), false);
  if (need) {
    CHECK_PTR(ws);
    if (ws_bytes < need)
      return fail(INFV2_E_WORKSPACE, "dense_attn workspace %zu < %zu bytes", ws_bytes, need);
  }
  return hip_status(launch_attn(*p, Q, K, V, nullptr, nullptr, O, lse, ws, budget_of(*p),
                                kv_cap_of(*p), scale_of(*p), (hipStream_t)stream),
                    "infv2_dense_attn");
}

size_t infv2_sparse_attn_bwd_workspace(const infv2_problem* p) {
  if (check(p) != INFV2_OK) return 0;
  return attn_bwd_workspace(*p, true);
}

size_t infv2_dense_attn_bwd_workspace(const infv2_problem* p) {
  if (check(p) != INFV2_OK) return 0;
  return attn_bwd_workspace(*p, false);
}

static int attn_bwd_common(const infv2_problem* p, const void* Q, const void* K, const void* V,
                           const int32_t* idx, const int32_t* n_sel, const void* O,
                           const float* lse, const void* dO, float* dQ, float* dK, float* dV,
                           void* ws, size_t ws_bytes, void* stream, const char* what) {
  int st = check(p);
  if (st) return st;
  const bool sparse = idx != nullptr;
  CHECK_PTR(Q);
  CHECK_PTR(K);
  CHECK_PTR(V);
  CHECK_PTR(O);
  CHECK_PTR(lse);
  CHECK_PTR(dO);
  CHECK_PTR(dQ);
  CHECK_PTR(dK);
  CHECK_PTR(dV);
  if (sparse) CHECK_PTR(n_sel);
  if (!attn_fast_shape(*p) && attn_bwd_generic_lds(*p, budget_of(*p), sparse) > 64 * 1024)
    return fail(INFV2_E_UNSUPPORTED,
                "%s: %s for the generic backward kernel (shape G=%d d=%d dtype=%d)", what,
                sparse ? "budget * B too large" : "n_kv too large", p->G, p->d, p->dtype);
  // the fast kernels launch (window, key block, batch * h_kv) grids and
  // (key block, h_kv, batch) pack grids: y and z hold at most 65535
  // (the sparse dK/dV grid adds 7 sub-windows per init block to y)
  if (attn_fast_shape(*p) &&
      ((int64_t)n_blk_of(*p) + 7 * (int64_t)p->N_init > 65535 || (int64_t)p->batch * p->h_kv > 65535))
    return fail(INFV2_E_UNSUPPORTED,
                "%s: ceil(n_kv/B) + 7 N_init (%lld) and batch x h_kv (%lld) must be at most 65535",
                what, (long long)n_blk_of(*p) + 7LL * p->N_init, (long long)p->batch * p->h_kv);
  const size_t need = attn_bwd_workspace(*p, sparse);
  if (need) {
    CHECK_PTR(ws);
    if (ws_bytes < need) return fail(INFV2_E_WORKSPACE, "%s workspace %zu < %zu bytes", what, ws_bytes, need);
  }
  return hip_status(launch_attn_bwd(*p, Q, K, V, idx, n_sel, O, lse, dO, dQ, dK, dV, ws,
                                    budget_of(*p), kv_cap_of(*p), scale_of(*p),
                                    (hipStream_t)stream),
                    what);
}

int infv2_sparse_attn_bwd(const infv2_problem* p, const void* Q, const void* K, const void* V,
                          const int32_t* idx, const int32_t* n_sel, const void* O,
                          const float* lse, const void* dO, float* dQ, float* dK, float* dV,
                          void* ws, size_t ws_bytes, void* stream) {
  if (!idx) return fail(INFV2_E_ARG, "idx is NULL");
  return attn_bwd_common(p, Q, K, V, idx, n_sel, O, lse, dO, dQ, dK, dV, ws, ws_bytes, stream,
                         "infv2_sparse_attn_bwd");
}

int infv2_dense_attn_bwd(const infv2_problem* p, const void* Q, const void* K, const void* V,
                         const void* O, const float* lse, const void* dO, float* dQ, float* dK,
                         float* dV, void* ws, size_t ws_bytes, void* stream) {
  return attn_bwd_common(p, Q, K, V, nullptr, nullptr, O, lse, dO, dQ, dK, dV, ws, ws_bytes,
                         stream, "infv2_dense_attn_bwd");
}

// ---- varlen batches / paged cache (decode shapes)
static int check_varlen(const infv2_problem* p, const char* what) {
  int st = check(p);
  if (st) return st;
  if (!scores_use_split(*p) || !attn_use_split(*p))
    return fail(INFV2_E_UNSUPPORTED,
                "%s: decode shapes only (bf16, G=16, d=128, B=64, l_C1=32, s_C1=16, n_q<=4)",
                what);
  if (!select_fused_shape(*p, n_c1_of(*p)))
    return fail(INFV2_E_UNSUPPORTED, "%s: needs k <= 32, budget <= 64 and n_kv <= 262144", what);
  return INFV2_OK;
}

static int check_pages(const infv2_problem& p, const int32_t* block_table, int32_t max_blocks,
                       int32_t n_pages) {
  if (!block_table) return INFV2_OK;
  CHECK_PTR(block_table);
  if (max_blocks < n_blk_of(p))
    return fail(INFV2_E_ARG, "max_blocks (%d) < ceil(n_kv/B) (%d)", max_blocks, n_blk_of(p));
  if (n_pages < 1) return fail(INFV2_E_ARG, "n_pages must be >= 1");
  return INFV2_OK;
}

int infv2_compress_k_varlen(const infv2_problem* p, const void* K, const int32_t* block_table,
                            int32_t max_blocks, int32_t n_pages, const int32_t* seq_lens,
                            void* Kc, int32_t coarse, int32_t last_n, void* stream) {
  int st = check_varlen(p, "infv2_compress_k_varlen");
  if (st) return st;
  CHECK_PTR(K);
  CHECK_PTR(seq_lens);
  CHECK_PTR(Kc);
  if (coarse != 0 && coarse != 1) return fail(INFV2_E_ARG, "coarse must be 0 or 1");
  if ((st = check_pages(*p, block_table, max_blocks, n_pages))) return st;
  const int l_len = coarse ? l_c2_of(*p) : p->l_C1;
  const int s_len = coarse ? s_c2_of(*p) : p->s_C1;
  return hip_status(launch_compress_k_varlen(*p, K, block_table, max_blocks, n_pages, seq_lens,
                                             Kc, kv_cap_of(*p), coarse ? c2_cap_of(*p) : c1_cap_of(*p),
                                             l_len, s_len, last_n, (hipStream_t)stream),
                    "infv2_compress_k_varlen");
}

size_t infv2_select_blocks_varlen_workspace(const infv2_problem* p) {
  if (check(p) != INFV2_OK || !scores_use_split(*p)) return 0;
  const KeySet ks = keys_of(*p, nullptr, nullptr);
  return align256(scores_workspace(*p, ks)) + select_fused_workspace(*p, ks.n_c1);
}

int infv2_select_blocks_varlen(const infv2_problem* p, const void* Q, const void* Kc1,
                               const void* Kc2, const int32_t* seq_lens, int32_t* idx,
                               int32_t* n_sel, void* ws, size_t ws_bytes, void* stream) {
  int st = check_varlen(p, "infv2_select_blocks_varlen");
  if (st) return st;
  CHECK_PTR(Q);
  CHECK_PTR(seq_lens);
  CHECK_PTR(idx);
  CHECK_PTR(n_sel);
  if ((st = check_keys(*p, Kc1, Kc2))) return st;
  const KeySet ks = keys_of(*p, Kc1, Kc2);
  const size_t need = infv2_select_blocks_varlen_workspace(p);
  CHECK_PTR(ws);
  if (ws_bytes < need)
    return fail(INFV2_E_WORKSPACE, "select_blocks_varlen workspace %zu < %zu bytes", ws_bytes,
                need);
  return hip_status(launch_select_varlen(*p, Q, ks, seq_lens, idx, n_sel, ws, n_blk_of(*p),
                                         scale_of(*p), budget_of(*p), (hipStream_t)stream),
                    "infv2_select_blocks_varlen");
}

size_t infv2_sparse_attn_varlen_workspace(const infv2_problem* p) {
  if (check(p) != INFV2_OK || !attn_use_split(*p)) return 0;
  return attn_workspace(*p, budget_of(*p), true);
}

int infv2_sparse_attn_varlen(const infv2_problem* p, const void* Q, const void* K, const void* V,
                             const int32_t* block_table, int32_t max_blocks, int32_t n_pages,
                             const int32_t* seq_lens, const int32_t* idx, const int32_t* n_sel,
                             void* O, float* lse, void* ws, size_t ws_bytes, void* stream) {
  int st = check_varlen(p, "infv2_sparse_attn_varlen");
  if (st) return st;
  CHECK_PTR(Q);
  CHECK_PTR(K);
  CHECK_PTR(V);
  CHECK_PTR(seq_lens);
  CHECK_PTR(idx);
  CHECK_PTR(n_sel);
  CHECK_PTR(O);
  if (lse && !aligned16(lse)) return fail(INFV2_E_ARG, "lse is not 16-byte aligned");
  if ((st = check_pages(*p, block_table, max_blocks, n_pages))) return st;
  const size_t need = infv2_sparse_attn_varlen_workspace(p);
  CHECK_PTR(ws);
  if (ws_bytes < need)
    return fail(INFV2_E_WORKSPACE, "sparse_attn_varlen workspace %zu < %zu bytes", ws_bytes, need);
  return hip_status(launch_attn_varlen(*p, Q, K, V, block_table, max_blocks, n_pages, seq_lens,
                                       idx, n_sel, O, lse, ws, budget_of(*p), kv_cap_of(*p),
                                       scale_of(*p), (hipStream_t)stream),
                    "infv2_sparse_attn_varlen");
}

const char* infv2_status_string(int status) {
  switch (status) {
    case INFV2_OK: return "ok";
    case INFV2_E_ARG: return "invalid argument";
    case INFV2_E_UNSUPPORTED: return "unsupported problem";
    case INFV2_E_WORKSPACE: return "workspace too small";
    case INFV2_E_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char* infv2_last_error(void) { return g_last_error.c_str(); }

#ifndef INFV2_SOURCE_HASH
#define INFV2_SOURCE_HASH "unknown"
#endif
const char* infv2_build_id(void) { return INFV2_SOURCE_HASH; }

}  // extern "C"
