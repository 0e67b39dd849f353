// Stages 2-3 of block selection: compressed scores, head-group sum, max-pool.
//
// papernotes.org InfLLM-V2 note, 方法详解 > 关键设计 3 (S^C1 = Softmax(Q K^C1^T),
// S^shared = sum over the G heads of a group, S^cmp = max-pool with l, s) and
// 关键设计 4 (fused head-group summation: S^C1 never reaches HBM; the normaliser
// comes from an exact log-sum-exp computed in an earlier sweep).  OpenBMB blog
// "技术Blog-4 | 新一代InfLLM：可训练的稀疏注意力机制", 动态上下文块选择 > 语义核 (block
// score = max over the kernels intersecting the block) and 高效Top-K实现.
//
// Three kernels:
//  * scores_prefill_kernel -- bf16, G = 16, d = 128, B = 64, l_C1 = 32,
//    s_C1 = 16.  One workgroup = 16 query tokens x 16 heads of one group (256
//    MFMA rows).  Q stays in registers; K^C1 streams through LDS in chunks of
//    32 kernels.  Two sweeps, as the pages describe: the first sums
//    2^(z*c - M) with M the exact row maximum of the first chunk (an extra
//    maximum sweep runs only if a later logit overflows that reference); the
//    second forms S^C1, sums the 16 heads (8 in-lane + one cross-half
//    exchange), max-pools into blocks and writes S^cmp.  S^C1 is never
//    written to memory; S^shared is written only by the SHARED instance,
//    when the caller passes a buffer for it.
//  * scores_split_{logits,pool}_kernel -- few query tokens (decode): the kernel
//    axis is split over workgroups; the first writes scaled logits and
//    per-chunk (max, sum) partials, the second merges the partials into the
//    exact log-sum-exp and forms S^shared / S^cmp for its chunk.
//  * scores_generic_kernel -- any shape and fp32 I/O: fp64 arithmetic, one
//    workgroup per (token, group).  Correctness path for the fp32 workload.
#include <type_traits>

#include "common.hpp"
#include "kc1_mean.hpp"
#include "select_merge.hpp"

namespace infv2 {

constexpr int SEL_D = 128;
constexpr int SEL_G = 16;
constexpr int SEL_CHUNK = 32;                 // kernels per LDS chunk (one MFMA N-tile)
constexpr int SEL_ROW_BYTES = SEL_D * 2;      // one K^C1 row, bf16
constexpr int SEL_TOK_WAVE = 4;               // tokens per wave (2 MFMA row blocks)
constexpr int SEL_TOK_WG = 16;                // tokens per workgroup

struct ScoresArgs {
  const uint16_t* Q;
  const uint16_t* Kc1;
  const uint16_t* Kc2;   // coarse keys (LSE approximation), else null
  float* S_cmp;          // null in the selection mode unless the caller wants it
  float* S_sh;           // S^shared [batch][h_kv][n_q][n_c1] when the caller wants it
  // selection mode (top-k streamed inside the score sweep): outputs, and one
  // mark per tile for the exact kernel (1: recompute this tile)
  int32_t* idx;
  int32_t* n_sel;
  int32_t* marks;        // [batch][h_kv][tiles]
  int k, N_init, N_local, budget;
  int batch, n_q, q_pos0, h_kv, n_c1, n_c2, n_blk, tiles;
  int64_t c1_cap, c2_cap;
  float c;  // scale * log2(e)
};

// ---------------------------------------------------------------------------
// Streaming top-k inside a wave, for NT query tokens.  Candidate blocks enter
// as 64-bit keys: order-preserving score bits << 32 | ~blk (unique; at equal
// scores the lower block ranks higher; 0 = no key).  A key that beats the
// token's threshold is appended to the token's 64-entry LDS buffer; when the
// buffer could overflow on the next push it is sorted by one wave and cut to
// its k best, whose k-th key becomes the threshold (keys are unique, so a key
// below it can never reach the final top k).  Buffer entries at and past the
// count are kept at 0.
// ---------------------------------------------------------------------------
template <int NT>
struct TopkStream {
  uint64_t tau[NT];   // keys <= tau are out (0 until k keys have been kept)
  int cnt[NT];        // keys in the token's buffer
};

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int l) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
  return ((uint64_t)hi << 32) | lo;
}

template <int NT>
__device__ __forceinline__ void topk_init(TopkStream<NT>& st, uint64_t* buf, int lane) {
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    st.tau[t] = 0ull;
    st.cnt[t] = 0;
    buf[t * 64 + lane] = 0ull;
  }
  wave_lds_sync();
}

// sort token t's buffer and keep its k best (all lanes active).  The pushes
// write the buffer without waiting; the waits are here, where it is read and
// rewritten (rarely: a few times per token).
template <int NT>
__device__ __forceinline__ void topk_compact(TopkStream<NT>& st, uint64_t* buf, int t, int lane,
                                             int k) {
  wave_lds_sync();
  const uint64_t sorted = wave_sort_desc<uint64_t>(buf[t * 64 + lane], lane);
  const int keep = min(st.cnt[t], k);
  wave_lds_sync();
  buf[t * 64 + lane] = lane < keep ? sorted : 0ull;
  st.cnt[t] = keep;
  if (keep > 0 && keep == k) st.tau[t] = readlane_u64(sorted, k - 1);
  wave_lds_sync();
}

// each lane offers at most one key (0: none) for its token tl; at most
// max_new keys per token per call (all lanes active)
template <int NT>
__device__ __forceinline__ void topk_push(TopkStream<NT>& st, uint64_t* buf, int tl, uint64_t key,
                                          int lane, int k, int max_new) {
  const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const bool hit = tl == t && key > st.tau[t];
    const uint64_t m = __ballot(hit);
    if (hit) buf[t * 64 + st.cnt[t] + (int)__popcll(m & below)] = key;
    st.cnt[t] += (int)__popcll(m);
  }
#pragma unroll
  for (int t = 0; t < NT; ++t)
    if (st.cnt[t] > 64 - max_new) topk_compact(st, buf, t, lane, k);
}

// Final selection of token t (after its last push): I(p) = init u local u
// the kept keys, ascending and -1 padded, to out[0..budget) (budget <= 64),
// and |I(p)| to *n_out.  Candidates lie strictly between the init and the
// local blocks, so the ascending set is init, then the kept blocks in
// ascending order, then local.
template <int NT>
__device__ __forceinline__ void topk_emit(TopkStream<NT>& st, uint64_t* buf, int t, int lane,
                                          int k, int p, int N_init, int N_local, int budget,
                                          int32_t* out, int32_t* n_out, bool write) {
  topk_compact(st, buf, t, lane, k);
  const int kk = st.cnt[t];
  const uint64_t key = buf[t * 64 + lane];
  const uint32_t nb_key = lane < kk ? (uint32_t)key : 0u;   // ~blk: larger = lower block
  const uint32_t asc = wave_sort_desc<uint32_t>(nb_key, lane);  // lanes 0..kk-1: ascending blocks
  const int b_p = p >> 6, nb = b_p + 1;
  const int init_hi = min(N_init, nb);
  const int loc_lo = max(0, b_p - N_local + 1);
  int v = -1, n;
  if (loc_lo <= init_hi) {             // init and local cover every causal block
    n = nb;
    v = lane < nb ? lane : -1;
  } else {
    n = init_hi + kk + (nb - loc_lo);
    const int blk_j = (int)~__shfl(asc, max(0, min(lane - init_hi, 63)), 64);
    if (lane < init_hi) v = lane;
    else if (lane < init_hi + kk) v = blk_j;
    else if (lane < n) v = loc_lo + (lane - init_hi - kk);
  }
  if (write) {
    if (lane < budget) out[lane] = v;
    if (lane == 0) *n_out = n;
  }
}

// kernel j is causal for position p when its last token j*16+31 <= p
__device__ __forceinline__ int last_visible_kernel(int p) { return p >= 31 ? (p - 31) >> 4 : -1; }
// coarse kernel j (tokens 64j .. 64j+127) is causal when 64j+127 <= p
__device__ __forceinline__ int last_visible_coarse(int p) { return p >= 127 ? (p - 127) >> 6 : -1; }
// log2(s_C2 / s_C1): the count correction of the coarse estimate
constexpr float kLog2CoarseRatio = 2.0f;

constexpr int PASS_MAX = 0;    // row maxima (only when the sum overflows)
constexpr int PASS_SUM = 1;    // log-sum-exp sweep
constexpr int PASS_SCORE = 2;  // normalised scores, group sum, max-pool


// Exact pass, one chunk of 32 kernels for the wave's 64 rows (4 tokens x 16
// heads), with a reference per row.
// MASKED chunks contain kernels that are not causal for some row.
//  PASS_MAX:   M = max(M, z)
//  PASS_SUM:   W += 2^(z*c - M); on the first chunk M is first set to the
//              chunk's exact row maximum (times c), the reference of the sum
//  PASS_SCORE: S^C1 = 2^(z*c - M) * W, summed over the group's 16 heads and
//              staged in sbuf for the max-pool
template <int PASS, bool MASKED>
__device__ __forceinline__ void exact_chunk(const ScoresArgs& a, const uint8_t* kb, int chunk,
                                             bool first, const bf16x8 (&qf)[2][8],
                                             const int (&jm)[4], float (&M)[2][16],
                                             float (&W)[2][16], float (&sbuf)[4][SEL_CHUNK + 1],
                                             int lane) {
  f32x16 acc[2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[rb][i] = 0.f;
  const int col = lane & 31;
  const int half = lane >> 5;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    const int c16 = 2 * ks + half;
    const u32x4 raw = *(const u32x4*)(kb + col * SEL_ROW_BYTES + ((c16 ^ (col & 15)) << 4));
    const bf16x8 bfrag = as_bf16x8(raw);
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) acc[rb] = mfma32(qf[rb][ks], bfrag, acc[rb]);
  }
  const int j = chunk * SEL_CHUNK + col;     // this lane's kernel
  // causal mask: only chunks that reach past a row's last visible kernel
  if constexpr (MASKED) {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (j > jm[2 * rb + (i >> 3)]) acc[rb][i] = kNegInf;
  }
  if constexpr (PASS == PASS_MAX) {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int i = 0; i < 16; ++i) M[rb][i] = fmaxf(M[rb][i], acc[rb][i]);
  } else if constexpr (PASS == PASS_SUM) {
    if (first) {
      // reference = exact maximum of this chunk's visible logits, per row
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float m = acc[rb][i];
#pragma unroll
          for (int o = 1; o < 32; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
          M[rb][i] = (m == kNegInf) ? 0.f : m * a.c;   // -inf rows: nothing visible
        }
    }
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int i = 0; i < 16; ++i) W[rb][i] += fast_exp2(__builtin_fmaf(acc[rb][i], a.c, -M[rb][i]));
  } else {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      float part0 = 0.f, part1 = 0.f;  // tokens 2rb and 2rb+1, this lane's 8 heads
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float e = fast_exp2(__builtin_fmaf(acc[rb][i], a.c, -M[rb][i]));
        if (i < 8) part0 = __builtin_fmaf(e, W[rb][i], part0);
        else       part1 = __builtin_fmaf(e, W[rb][i], part1);
      }
      // lanes l and l^32 hold the other 8 heads of the same (token, kernel)
      const float send = half ? part0 : part1;
      const float recv = __shfl_xor(send, 32, 64);
      const float mine = (half ? part1 : part0) + recv;
      const int tl = 2 * rb + half;
      sbuf[tl][1 + col] = (j > jm[tl]) ? kNegInf : mine;
    }
  }
}

// The exact pass: the same two sweeps with one exponent reference per row
// (and an extra maximum sweep when a sum overflows).  It runs only for the
// tiles that the fast kernel marked (NaN in block 0 of the tile's first row)
// and exits at once for all others.  APPROX: rows whose token sees a coarse
// kernel take the coarse estimate (a sum sweep over K^C2 with the same
// machinery), the others the exact LSE; the score sweep then uses
// 2^(z*c - L) with L = log2 of the row's normaliser.
// SELECT: the selection mode of the fast kernel (marks instead of the NaN
// marker; idx / n_sel from a streaming top-k; S^cmp only when a.S_cmp is set).
// The body is a separate (not inlined) function: most workgroups leave at
// the mark test, before the body's stack frame exists.
template <bool APPROX, bool SELECT>
__device__ __noinline__ void scores_exact_body(const ScoresArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t kbuf[2][SEL_CHUNK * SEL_ROW_BYTES];
  __shared__ float sbuf_all[4][SEL_TOK_WAVE][SEL_CHUNK + 1];
  __shared__ float lfine_all[4][2][32];   // APPROX: exact log2-normaliser per row
  __shared__ uint64_t tkbuf_all[SELECT ? 4 : 1][SEL_TOK_WAVE][64];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int bid = blockIdx.x;
  const int tile = bid % a.tiles;
  const int g = (bid / a.tiles) % a.h_kv;
  const int b = bid / (a.tiles * a.h_kv);
  TopkStream<SEL_TOK_WAVE> tk;
  uint64_t* tkbuf = &tkbuf_all[SELECT ? wave : 0][0][0];
  if constexpr (SELECT) topk_init<SEL_TOK_WAVE>(tk, tkbuf, lane);
  const int wg_t0 = tile * SEL_TOK_WG;
  const int t0 = wg_t0 + wave * SEL_TOK_WAVE;
  const int hq = a.h_kv * SEL_G;
  float (&sbuf)[4][SEL_CHUNK + 1] = sbuf_all[wave];

  // ---- Q fragments (A operand: rows = (token, head), k = d) ----
  bf16x8 qf[2][8];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int tok = t0 + 2 * rb + ((lane & 31) >> 4);
    const int head = g * SEL_G + (lane & 15);
    // rows of tokens past n_q read the last token; they are never written
    const uint16_t* qrow = a.Q + (((size_t)b * a.n_q + min(tok, a.n_q - 1)) * hq + head) * SEL_D;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[rb][ks] = as_bf16x8(*(const u32x4*)(qrow + 16 * ks + 8 * (lane >> 5)));
  }
  int jm[4];
#pragma unroll
  for (int tl = 0; tl < 4; ++tl) {
    const int tok = t0 + tl;
    jm[tl] = tok < a.n_q ? last_visible_kernel(a.q_pos0 + tok) : -1;
  }
  const int wg_last = min(wg_t0 + SEL_TOK_WG - 1, a.n_q - 1);
  const int jmax_wg = last_visible_kernel(a.q_pos0 + wg_last);
  const int jmin_wg = last_visible_kernel(a.q_pos0 + wg_t0);
  const int nchunks = jmax_wg < 0 ? 0 : (jmax_wg + 2 + SEL_CHUNK - 1) / SEL_CHUNK;

  float M[2][16], W[2][16];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int i = 0; i < 16; ++i) { M[rb][i] = kNegInf; W[rb][i] = 0.f; }

  const uint16_t* kc1 = a.Kc1 + ((size_t)b * a.h_kv + g) * a.c1_cap * SEL_D;
  // the sweep's key rows: K^C1, or K^C2 for the approximate LSE sweep
  const uint16_t* src = kc1;
  int n_src = a.n_c1;

  // stage one chunk of 32 key rows (8 KB): 2 x 16 B per thread, XOR-swizzled
  auto stage_load = [&](int chunk, u32x4 (&st)[2]) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int u = tid + 256 * i;
      const int row = u >> 4, c16 = u & 15;
      // rows past the last kernel are clamped to it; they are never visible
      const int j = min(chunk * SEL_CHUNK + row, n_src - 1);
      st[i] = *(const u32x4*)(src + (size_t)j * SEL_D + c16 * 8);
    }
  };
  auto stage_store = [&](uint8_t* kb, const u32x4 (&st)[2]) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int u = tid + 256 * i;
      const int row = u >> 4, c16 = u & 15;
      *(u32x4*)(kb + row * SEL_ROW_BYTES + ((c16 ^ (row & 15)) << 4)) = st[i];
    }
  };

  auto run_pass = [&](auto pass_tag, bool set_ref, int nchunks, int jmin_wg) {
    constexpr int PASS = decltype(pass_tag)::value;
    if (nchunks == 0) return;
    u32x4 st[2];
    stage_load(0, st);
    stage_store(kbuf[0], st);
    __syncthreads();
    for (int c = 0; c < nchunks; ++c) {
      const bool more = c + 1 < nchunks;
      if (more) stage_load(c + 1, st);
      const bool masked = c * SEL_CHUNK + SEL_CHUNK - 1 > jmin_wg;
      const bool first = set_ref && c == 0;
      if (masked)
        exact_chunk<PASS, true>(a, kbuf[c & 1], c, first, qf, jm, M, W, sbuf, lane);
      else
        exact_chunk<PASS, false>(a, kbuf[c & 1], c, first, qf, jm, M, W, sbuf, lane);
      if constexpr (PASS == PASS_SCORE) {
        // max-pool: block c*8+bb takes kernels c*32+4bb-1 .. c*32+4bb+3,
        // i.e. sbuf[tl][4bb .. 4bb+4] (sbuf[tl][0] carries kernel c*32-1);
        // lanes 0..31 hold the 4 tokens x 8 blocks of the chunk
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const int tl = (lane >> 3) & 3, bb = lane & 7;
        float v = sbuf[tl][4 * bb];
#pragma unroll
        for (int q = 1; q < 5; ++q) v = fmaxf(v, sbuf[tl][4 * bb + q]);
        const int tok = t0 + tl;
        const int blk = c * (SEL_CHUNK / 4) + bb;
        const int b_p = (a.q_pos0 + tok) >> 6;
        if (lane < 32 && a.S_cmp && tok < a.n_q && blk <= b_p)
          a.S_cmp[(((size_t)b * a.h_kv + g) * a.n_q + tok) * a.n_blk + blk] = v;
        if (!SELECT && a.S_sh) {
          // S^shared of the chunk's 32 kernels for the 4 tokens (0 where not seen)
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int u = lane + 64 * e, ut = u >> 5, x = u & 31;
            const int j = c * SEL_CHUNK + x;
            if (t0 + ut < a.n_q && j < a.n_c1) {
              const float sv = sbuf[ut][1 + x];
              a.S_sh[(((size_t)b * a.h_kv + g) * a.n_q + t0 + ut) * a.n_c1 + j] =
                  (sv == kNegInf) ? 0.f : sv;
            }
          }
        }
        if constexpr (SELECT) {
          const bool cand = lane < 32 && tok < a.n_q && blk >= min(a.N_init, b_p + 1) &&
                            blk < max(0, b_p - a.N_local + 1);
          const uint64_t key = cand ? ((uint64_t)ordered_bits(v) << 32) | (uint64_t)(~(uint32_t)blk)
                                    : 0ull;
          topk_push<SEL_TOK_WAVE>(tk, tkbuf, tl, key, lane, a.k, SEL_CHUNK / 4);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        if (lane < 4) sbuf[lane][0] = sbuf[lane][SEL_CHUNK];
      }
      if (more) stage_store(kbuf[(c + 1) & 1], st);
      __syncthreads();
    }
  };
  auto merge_sums = [&]() -> bool {   // lane partial sums -> row sums; true if finite
    bool ok = true;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float s = W[rb][i];
#pragma unroll
        for (int o = 1; o < 32; o <<= 1) s += __shfl_xor(s, o, 64);
        W[rb][i] = s;
        ok = ok && __builtin_isfinite(s);
      }
    return ok;
  };

  // sweep 1 (log-sum-exp): s = sum_j 2^(z_j*c - M), M = the exact row maximum
  // over the first chunk (every row with a visible kernel sees kernel 0)
  auto lse_sweep = [&](int nch, int jmin) {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int i = 0; i < 16; ++i) { M[rb][i] = kNegInf; W[rb][i] = 0.f; }
    run_pass(std::integral_constant<int, PASS_SUM>{}, true, nch, jmin);
    const bool finite = merge_sums();
    if (__syncthreads_or(!finite)) {
      // a later logit exceeded the reference by more than 2^127: take the
      // exact row maximum (one extra sweep) and sum again
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int i = 0; i < 16; ++i) { M[rb][i] = kNegInf; W[rb][i] = 0.f; }
      run_pass(std::integral_constant<int, PASS_MAX>{}, false, nch, jmin);
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float m = M[rb][i];
#pragma unroll
          for (int o = 1; o < 32; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
          M[rb][i] = (m == kNegInf) ? 0.f : m * a.c;
        }
      run_pass(std::integral_constant<int, PASS_SUM>{}, false, nch, jmin);
      merge_sums();
    }
  };
  if constexpr (!APPROX) {
    lse_sweep(nchunks, jmin_wg);
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int i = 0; i < 16; ++i) W[rb][i] = W[rb][i] > 0.f ? 1.0f / W[rb][i] : 0.f;
  } else {
    // Row (rb, i) of this lane is token 2rb + (row >> 4), head row & 15, with
    // row = 8(i/4) + 4(lane/32) + i%4 (32x32 C layout); after merge_sums its
    // M and W are the same in the 32 lanes of the lane's half.
    auto row_of = [&](int i) { return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3); };
    const int p_first = a.q_pos0 + wg_t0, p_last = a.q_pos0 + wg_last;
    const bool need_fine = p_first < 127 && p_last >= 31;
    if (need_fine) {
      // exact normaliser of the tokens that see no coarse kernel
      lse_sweep(nchunks, jmin_wg);
      if ((lane & 31) == 0)
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            lfine_all[wave][rb][row_of(i)] = M[rb][i] + fast_log2(W[rb][i]);
    }
    int jm2[4];
#pragma unroll
    for (int tl = 0; tl < 4; ++tl) jm2[tl] = t0 + tl < a.n_q ? last_visible_coarse(a.q_pos0 + t0 + tl) : -1;
    const int jmax2 = last_visible_coarse(p_last), jmin2 = last_visible_coarse(p_first);
    if (jmax2 >= 0) {
      // coarse sweep (masks from the coarse visibility)
      int jm_fine[4];
#pragma unroll
      for (int tl = 0; tl < 4; ++tl) { jm_fine[tl] = jm[tl]; jm[tl] = jm2[tl]; }
      src = a.Kc2 + ((size_t)b * a.h_kv + g) * a.c2_cap * SEL_D;
      n_src = a.n_c2;
      lse_sweep((jmax2 + SEL_CHUNK) / SEL_CHUNK, jmin2);
      src = kc1;
      n_src = a.n_c1;
#pragma unroll
      for (int tl = 0; tl < 4; ++tl) jm[tl] = jm_fine[tl];
    }
    __syncthreads();
    // per row: L = coarse estimate where the token sees a coarse kernel,
    // else the exact one; the score sweep runs with M = L and W = 1
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int tl = 2 * rb + (row_of(i) >> 4);
        const float l2 = M[rb][i] + (fast_log2(W[rb][i]) + kLog2CoarseRatio);
        M[rb][i] = jm2[tl] >= 0 ? l2 : (need_fine ? lfine_all[wave][rb][row_of(i)] : 0.f);
        W[rb][i] = 1.0f;
      }
  }
  // sweep 2: S^C1 = 2^(z*c - M) / s, head-group sum, max-pool, S^cmp
  if (lane < 4) sbuf[lane][0] = kNegInf;
  run_pass(std::integral_constant<int, PASS_SCORE>{}, false, nchunks, jmin_wg);
  // blocks with no visible kernel in the causal range
  if (a.S_cmp) {
    const int tl = lane >> 4;
    const int tok = t0 + tl;
    if (tok < a.n_q) {
      const int b_p = (a.q_pos0 + tok) >> 6;
      float* row = a.S_cmp + (((size_t)b * a.h_kv + g) * a.n_q + tok) * a.n_blk;
      for (int blk = nchunks * (SEL_CHUNK / 4) + (lane & 15); blk <= b_p; blk += 16)
        row[blk] = kNegInf;
    }
  }
  if (!SELECT && a.S_sh) {   // S^shared past the swept chunks
    const int tok = t0 + (lane >> 4);
    if (tok < a.n_q) {
      float* row = a.S_sh + (((size_t)b * a.h_kv + g) * a.n_q + tok) * a.n_c1;
      for (int j = nchunks * SEL_CHUNK + (lane & 15); j < a.n_c1; j += 16) row[j] = 0.f;
    }
  }
  if constexpr (SELECT) {
#pragma unroll
    for (int tl = 0; tl < SEL_TOK_WAVE; ++tl) {
      const int tok = t0 + tl;
      const size_t row = ((size_t)b * a.h_kv + g) * a.n_q + min(tok, a.n_q - 1);
      topk_emit<SEL_TOK_WAVE>(tk, tkbuf, tl, lane, a.k, a.q_pos0 + min(tok, a.n_q - 1),
                              a.N_init, a.N_local, a.budget, a.idx + row * a.budget,
                              a.n_sel + row, tok < a.n_q);
    }
  }
}

template <bool APPROX, bool SELECT>
__global__ void __launch_bounds__(256, 2) scores_exact_kernel(ScoresArgs a) {
  const int bid = blockIdx.x;
  const int tile = bid % a.tiles;
  const int g = (bid / a.tiles) % a.h_kv;
  const int b = bid / (a.tiles * a.h_kv);
  if constexpr (SELECT) {
    if (a.marks[((size_t)b * a.h_kv + g) * a.tiles + tile] == 0) return;
  } else {
    const float mark = a.S_cmp[(((size_t)b * a.h_kv + g) * a.n_q + tile * SEL_TOK_WG) * a.n_blk];
    if (!__builtin_isnan(mark)) return;
  }
  scores_exact_body<APPROX, SELECT>(a);
}

constexpr int SEL_DEPTH = 4;                                // K^C1 chunks in flight per wave
constexpr int SEL_CHUNK_BYTES = SEL_CHUNK * SEL_ROW_BYTES;  // 8 KB
constexpr int FAST_TOK_WAVE = 2;                            // tokens per wave
constexpr int FAST_WAVES = SEL_TOK_WG / FAST_TOK_WAVE;      // 8 waves, 512 threads

// Lane moves by the data-parallel primitives.  Every cross-lane read runs
// with all lanes active (a read from an inactive lane yields 0).
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}
constexpr int DPP_QUAD_XOR1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int DPP_QUAD_XOR2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int DPP_QUAD_BC0 = 0x00;    // quad_perm [0,0,0,0]
constexpr int DPP_WAVE_SHR1 = 0x138;  // lane l <- lane l-1

// Sum of four per-lane values A, B, C, D over the four 16-lane rows (lanes
// l, l^16, l^32, l^48).  Lanes of row 0 receive A's sum, row 1 C's, row 2
// B's, row 3 D's (two permlane32 swaps, then one permlane16 swap).
__device__ __forceinline__ float row_sum4(float A, float B, float C, float D) {
  const auto s1 = __builtin_amdgcn_permlane32_swap(__float_as_uint(A), __float_as_uint(B), false, false);
  const auto s2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(C), __float_as_uint(D), false, false);
  const float r1 = __uint_as_float(s1[0]) + __uint_as_float(s1[1]);   // rows 0,1: A; rows 2,3: B
  const float r2 = __uint_as_float(s2[0]) + __uint_as_float(s2[1]);   // rows 0,1: C; rows 2,3: D
  const auto s3 = __builtin_amdgcn_permlane16_swap(__float_as_uint(r1), __float_as_uint(r2), false, false);
  return __uint_as_float(s3[0]) + __uint_as_float(s3[1]);
}

// Register state of one wave: 2 query tokens x 16 heads.  MFMA tiles are
// 16x16x32: token tl's 16 heads are the M rows, 16 kernels the N columns;
// acc[tl][nt] holds kernels 16nt .. 16nt+15 of the chunk.  In the C layout
// lane l holds heads 4*(l>>4) + i (i = 0..3) of column l&15.  After the head
// sum, lane row r = l>>4 holds token r>>1, kernels 16*(r&1) + (l&15).
struct SelWave {
  bf16x8 qf[2][4];   // A operand per token and k-step: head l&15, d = 32ks + 8(l>>4) ..+7
  float Mt[2];       // exponent reference per token (times c, wave-uniform)
  float W[2][4];     // PASS_SUM: partial sums; PASS_SCORE: 1 / row sum; [token][i]
  float carry;       // PASS_SCORE: S^shared of kernel (chunk start - 1), rows 0 and 2
  int jm[2];         // last visible kernel per token (wave-uniform)
  int jm_l;          // the same for the token of this lane's row after the head sum
  int bp_l;          // its last causal block
  float* srow;       // its S^cmp row (null: not written)
  float* shrow;      // its S^shared row (SHARED kernels only)
  TopkStream<2> tk;  // selection mode: streaming top-k of the wave's 2 tokens
  uint64_t* tkbuf;   // their LDS buffers [2][64]
};

// z = Q K^C1^T for one chunk of 32 kernels staged in LDS (16-byte piece c of
// row r stored at piece position c ^ (r & 15)).
__device__ __forceinline__ void chunk_mfma(const uint8_t* kb, const SelWave& w, int lane,
                                           f32x4 (&acc)[2][2]) {
  const int r16 = lane & 15, grp = lane >> 4;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int row = nt * 16 + r16;
      const int piece = 4 * ks + grp;
      const bf16x8 bfrag = as_bf16x8(*(const u32x4*)(kb + row * SEL_ROW_BYTES + ((piece ^ r16) << 4)));
#pragma unroll
      for (int tl = 0; tl < 2; ++tl)
        acc[tl][nt] = mfma16(w.qf[tl][ks], bfrag, ks == 0 ? f32x4{} : acc[tl][nt]);
    }
  }
}

// Vector work on the logits z of chunk `chunk`.  MASKED chunks contain
// kernels that are not causal for some token.  The exponent reference M is
// per token (its 16 heads share it):
//  PASS_SUM:   W += 2^(z*c - M); FIRST: M is first set to the exact maximum
//              of the chunk's logits over the token's 16 heads (times c)
//  PASS_SCORE: S^C1 = 2^(z*c - M) * W (LFORM: 2^(z*c - W), W holding each
//              head's log2-normaliser), summed over the group's 16 heads,
//              max-pooled over the kernels that intersect each block and
//              written to S^cmp; SHR: S^shared itself is written as well
//              (0 for the kernels the token does not see)
template <int PASS, bool MASKED, bool FIRST, bool LFORM = false, bool TOPK = false,
          bool SHR = false>
__device__ __forceinline__ void chunk_valu(const ScoresArgs& a, f32x4 (&acc)[2][2], int chunk,
                                           SelWave& w, int lane) {
  static_assert(PASS == PASS_SUM || PASS == PASS_SCORE, "fast passes");
  const int r16 = lane & 15;
  if constexpr (MASKED) {
#pragma unroll
    for (int tl = 0; tl < 2; ++tl)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const bool out = chunk * SEL_CHUNK + nt * 16 + r16 > w.jm[tl];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (out) acc[tl][nt][i] = kNegInf;
      }
  }
  if constexpr (PASS == PASS_SUM) {
    if constexpr (FIRST) {
#pragma unroll
      for (int tl = 0; tl < 2; ++tl) {
        float m = acc[tl][0][0];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
          for (int i = 0; i < 4; ++i) m = fmaxf(m, acc[tl][nt][i]);
        m = wave_max(m);
        m = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(m)));
        w.Mt[tl] = (m == kNegInf) ? 0.f : m * a.c;   // -inf: nothing visible
      }
    }
#pragma unroll
    for (int tl = 0; tl < 2; ++tl)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          w.W[tl][i] += fast_exp2(__builtin_fmaf(acc[tl][nt][i], a.c, -w.Mt[tl]));
  } else {
    float part[2][2];   // [token][nt]: this lane's 4 heads
#pragma unroll
    for (int tl = 0; tl < 2; ++tl)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if constexpr (LFORM)
            s += fast_exp2(__builtin_fmaf(acc[tl][nt][i], a.c, -w.W[tl][i]));
          else
            s = __builtin_fmaf(fast_exp2(__builtin_fmaf(acc[tl][nt][i], a.c, -w.Mt[tl])),
                               w.W[tl][i], s);
        }
        part[tl][nt] = s;
      }
    // rows 0..3 <- (token 0, nt 0), (token 0, nt 1), (token 1, nt 0), (token 1, nt 1)
    float v = row_sum4(part[0][0], part[1][0], part[0][1], part[1][1]);
    const int nt = (lane >> 4) & 1;
    if constexpr (MASKED) v = (chunk * SEL_CHUNK + nt * 16 + r16 > w.jm_l) ? kNegInf : v;
    if constexpr (SHR) {
      const int j = chunk * SEL_CHUNK + nt * 16 + r16;
      if (j < a.n_c1) w.shrow[j] = (v == kNegInf) ? 0.f : v;
    }
    // block bb = 4nt + r16/4 of the chunk takes kernels 4bb-1 .. 4bb+3: the
    // max over its quad of lanes and the kernel before it (the previous lane;
    // for rows 0 and 2 at column 0, the last kernel of the previous chunk)
    float q = fmaxf(v, dpp<DPP_QUAD_XOR1>(v));
    q = fmaxf(q, dpp<DPP_QUAD_XOR2>(q));
    const float shr = dpp<DPP_WAVE_SHR1>(v);
    const float prev = (r16 == 0 && nt == 0) ? w.carry : shr;
    const float bv = fmaxf(q, dpp<DPP_QUAD_BC0>(prev));   // same in all 4 lanes of the quad
    const int blk = chunk * (SEL_CHUNK / 4) + nt * 4 + (r16 >> 2);
    if (w.srow && (!MASKED || blk <= w.bp_l)) __builtin_nontemporal_store(bv, w.srow + blk);
    if constexpr (TOPK) {
      // one lane of each quad offers the block when it is a candidate
      const int init_hi = min(a.N_init, w.bp_l + 1);
      const int loc_lo = max(0, w.bp_l - a.N_local + 1);
      const bool cand = (r16 & 3) == 0 && blk >= init_hi && blk < loc_lo;
      const uint64_t key = cand ? ((uint64_t)ordered_bits(bv) << 32) | (uint64_t)(~(uint32_t)blk)
                                : 0ull;
      topk_push<2>(w.tk, w.tkbuf, lane >> 5, key, lane, a.k, SEL_CHUNK / 4);
    }
    // kernel 31 of this chunk: lane 31 (token 0) and lane 63 (token 1)
    const float k31_t0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 31));
    const float k31_t1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
    w.carry = lane < 32 ? k31_t0 : k31_t1;
  }
}

// SELECT: the selection mode.  Each wave streams the top-k of its two tokens
// through the score sweep (no S^cmp round trip; S^cmp is still written when
// a.S_cmp is set) and writes idx / n_sel; the tile's mark tells the exact
// kernel whether to redo it.  SHARED: S^shared is written to a.S_sh too (a
// separate instance, so that the others keep their registers).
template <bool APPROX, bool SELECT, bool SHARED = false>
__global__ void __launch_bounds__(512, 4) scores_prefill_kernel(ScoresArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t kbuf[2 * SEL_CHUNK_BYTES];
  __shared__ uint64_t tkbuf_all[SELECT ? FAST_WAVES : 1][2][64];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  // Workgroups go round-robin over the 8 XCDs.  With h_kv dividing 8, XCD x
  // takes only group x % h_kv, so each XCD's L2 holds one group's K^C1;
  // within a group, tiles run from the last (longest rows) to the first.
  int tile, g, b;
  {
    const int bid = blockIdx.x;
    if (8 % a.h_kv == 0) {
      const int xcd = bid & 7, r = bid >> 3;
      const int per = 8 / a.h_kv;                      // XCDs per group
      g = xcd % a.h_kv;
      const int wi = r * per + xcd / a.h_kv;           // work index within the group
      if (wi >= a.tiles * a.batch) return;
      b = wi % a.batch;
      tile = a.tiles - 1 - wi / a.batch;
    } else {
      if (bid >= a.tiles * a.batch * a.h_kv) return;
      tile = a.tiles - 1 - (bid % a.tiles);
      const int bg = bid / a.tiles;
      g = bg % a.h_kv;
      b = bg / a.h_kv;
    }
  }
  const int wg_t0 = tile * SEL_TOK_WG;
  const int t0 = wg_t0 + wave * FAST_TOK_WAVE;
  const int hq = a.h_kv * SEL_G;
  float* srows = a.S_cmp ? a.S_cmp + ((size_t)b * a.h_kv + g) * a.n_q * a.n_blk : nullptr;
  const size_t tile_id = ((size_t)b * a.h_kv + g) * a.tiles + tile;
  // hands the tile to the exact kernel
  auto mark_tile = [&]() {
    if (tid == 0) {
      if constexpr (SELECT) a.marks[tile_id] = 1;
      else srows[(size_t)wg_t0 * a.n_blk] = __builtin_nanf("");
    }
  };

  // Tokens past n_q (ragged last tile) repeat the last token: they compute
  // its values and write them to its row again.
  SelWave w;
#pragma unroll
  for (int tl = 0; tl < 2; ++tl) {
    const int tok = min(t0 + tl, a.n_q - 1);
    const uint16_t* qrow = a.Q + (((size_t)b * a.n_q + tok) * hq + g * SEL_G + (lane & 15)) * SEL_D;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      w.qf[tl][ks] = as_bf16x8(__builtin_nontemporal_load((const u32x4*)(qrow + 32 * ks + 8 * (lane >> 4))));
    w.jm[tl] = last_visible_kernel(a.q_pos0 + tok);
  }
  {
    const int tok = min(t0 + (lane >> 5), a.n_q - 1);
    w.jm_l = last_visible_kernel(a.q_pos0 + tok);
    w.bp_l = (a.q_pos0 + tok) >> 6;
    w.srow = srows ? srows + (size_t)tok * a.n_blk : nullptr;
    if constexpr (SHARED) w.shrow = a.S_sh + (((size_t)b * a.h_kv + g) * a.n_q + tok) * a.n_c1;
  }
  if constexpr (SELECT) {
    w.tkbuf = &tkbuf_all[wave][0][0];
    topk_init<2>(w.tk, w.tkbuf, lane);
  }
  const int wg_last = min(wg_t0 + SEL_TOK_WG - 1, a.n_q - 1);
  const int jmax_wg = last_visible_kernel(a.q_pos0 + wg_last);
  const int jmin_wg = last_visible_kernel(a.q_pos0 + wg_t0);
  const int nchunks = jmax_wg < 0 ? 0 : (jmax_wg + 2 + SEL_CHUNK - 1) / SEL_CHUNK;
  // chunks below n_full hold only kernels that every row of the workgroup sees
  const int n_full = jmin_wg < 0 ? 0 : (jmin_wg + 1) / SEL_CHUNK;

#pragma unroll
  for (int tl = 0; tl < 2; ++tl) {
    w.Mt[tl] = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) w.W[tl][i] = 0.f;
  }

  const uint16_t* kc1 = a.Kc1 + ((size_t)b * a.h_kv + g) * a.c1_cap * SEL_D;

  // The LSE approximation takes the normaliser from the coarse kernels.  A
  // tile holding a token that sees fine kernels but no coarse kernel (it
  // keeps the exact LSE) goes to the exact kernel.
  if constexpr (APPROX) {
    if (a.q_pos0 + wg_t0 < 127 && a.q_pos0 + wg_last >= 31) {
      mark_tile();
      return;
    }
  }

  // K^C1 streams through LDS in chunks of 32 kernels (8 KB): 512 pieces of
  // 16 bytes, one per lane of the 8 waves.  Lane L of wave w owns piece
  // u = 64 w + L, i.e. row u/16 at piece position u%16, which holds global
  // piece (u%16) ^ (row & 15) of that row.  Each wave keeps the pieces of
  // the next SEL_DEPTH chunks in flight in registers (plain loads, so that
  // the compiler tracks each register's wait); a chunk goes to LDS one step
  // before it is used.  Chunks past the last one re-load the last kernel.
  const int piece_u = wave * 64 + lane;
  const int piece_row = piece_u >> 4;
  const uint32_t piece_src = (uint32_t)((((piece_u & 15) ^ (piece_row & 15)) << 3));   // elements
  uint8_t* const piece_dst = kbuf + piece_u * 16;
  // the sweep's key rows: K^C1, or K^C2 for the approximate LSE sweep
  const uint16_t* src = kc1;
  int n_src = a.n_c1;
  auto load_piece = [&](int c) -> u32x4 {
    const int j = min(c * SEL_CHUNK + piece_row, n_src - 1);
    return *(const u32x4*)(src + (size_t)j * SEL_D + piece_src);
  };
  auto slot = [&](int c) -> const uint8_t* { return kbuf + (c & 1) * SEL_CHUNK_BYTES; };

  // One sweep.  Step c: logits and vector work of chunk c (slot c & 1), then
  // chunk c+1 from registers into the other slot, the register refilled with
  // chunk c+1+SEL_DEPTH, and the barrier that publishes chunk c+1.
  auto run_pass = [&](auto pass_tag, auto ref_tag, int nchunks, int n_full) {
    constexpr int PASS = decltype(pass_tag)::value;
    constexpr bool SET_REF = decltype(ref_tag)::value;
    if (nchunks == 0) return;
    u32x4 st[SEL_DEPTH];
#pragma unroll
    for (int k = 0; k < SEL_DEPTH; ++k) st[k] = load_piece(k);
    *(u32x4*)piece_dst = st[0];
    st[0] = load_piece(SEL_DEPTH);
    __syncthreads();
    auto step = [&](int c, u32x4& next) {
      f32x4 acc[2][2];
      chunk_mfma(slot(c), w, lane, acc);
      constexpr bool LF = APPROX && PASS == PASS_SCORE;
      constexpr bool TK = SELECT && PASS == PASS_SCORE;
      constexpr bool SH = SHARED && PASS == PASS_SCORE;
      if (SET_REF && c == 0) {
        if (n_full > 0) chunk_valu<PASS, false, SET_REF, LF, TK, SH>(a, acc, c, w, lane);
        else            chunk_valu<PASS, true, SET_REF, LF, TK, SH>(a, acc, c, w, lane);
      } else if (c < n_full) {
        chunk_valu<PASS, false, false, LF, TK, SH>(a, acc, c, w, lane);
      } else {
        chunk_valu<PASS, true, false, LF, TK, SH>(a, acc, c, w, lane);
      }
      *(u32x4*)(piece_dst + ((c + 1) & 1) * SEL_CHUNK_BYTES) = next;
      next = load_piece(c + 1 + SEL_DEPTH);
      __syncthreads();
    };
    static_assert(SEL_DEPTH == 4, "unrolled below");
    int c = 0;
    for (; c + 4 <= nchunks; c += 4) {
      step(c, st[1]);
      step(c + 1, st[2]);
      step(c + 2, st[3]);
      step(c + 3, st[0]);
    }
    if (c < nchunks) step(c, st[1]);
    if (c + 1 < nchunks) step(c + 1, st[2]);
    if (c + 2 < nchunks) step(c + 2, st[3]);
  };

  // sweep 1 (log-sum-exp): s = sum_j 2^(z_j*c - M), M = the exact maximum
  // over the first chunk and the token's 16 heads (every row with a visible
  // kernel sees kernel 0).  APPROX: the same over the coarse kernels.
  if constexpr (APPROX) {
    src = a.Kc2 + ((size_t)b * a.h_kv + g) * a.c2_cap * SEL_D;
    n_src = a.n_c2;
    int jm_fine[2];
#pragma unroll
    for (int tl = 0; tl < 2; ++tl) {
      jm_fine[tl] = w.jm[tl];
      w.jm[tl] = last_visible_coarse(a.q_pos0 + min(t0 + tl, a.n_q - 1));
    }
    const int jmax2 = last_visible_coarse(a.q_pos0 + wg_last);
    const int jmin2 = last_visible_coarse(a.q_pos0 + wg_t0);
    run_pass(std::integral_constant<int, PASS_SUM>{}, std::true_type{},
             jmax2 < 0 ? 0 : (jmax2 + SEL_CHUNK) / SEL_CHUNK,
             jmin2 < 0 ? 0 : (jmin2 + 1) / SEL_CHUNK);
#pragma unroll
    for (int tl = 0; tl < 2; ++tl) w.jm[tl] = jm_fine[tl];
    src = kc1;
    n_src = a.n_c1;
  } else {
    run_pass(std::integral_constant<int, PASS_SUM>{}, std::true_type{}, nchunks, n_full);
  }
  // Lane partial sums -> row sums (over the 16 columns of a lane row).  A
  // row whose sum overflowed (a later logit exceeds the reference by more
  // than 2^127) or fell below 2^-64 (its head lies far below the token's
  // other heads, so that terms could underflow) sends the whole tile to the
  // exact kernel, which takes one reference per row.
  bool bad = false;
#pragma unroll
  for (int tl = 0; tl < 2; ++tl)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float s = w.W[tl][i];
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) s += __shfl_xor(s, o, 64);
      if constexpr (APPROX)   // log2 of the normaliser: M + log2(s) + log2(s_C2/s_C1)
        w.W[tl][i] = w.Mt[tl] + (fast_log2(s) + kLog2CoarseRatio);
      else
        w.W[tl][i] = s > 0.f ? 1.0f / s : 0.f;
      bad = bad || (w.jm[tl] >= 0 && !(s >= 0x1p-64f && s <= 0x1p127f));
    }
  if (__syncthreads_or(bad)) {
    mark_tile();
    return;
  }
  // sweep 2: S^C1 = 2^(z*c - M) / s (APPROX: 2^(z*c - L)), head-group sum,
  // max-pool, S^cmp
  w.carry = kNegInf;
  run_pass(std::integral_constant<int, PASS_SCORE>{}, std::false_type{}, nchunks, n_full);
  // blocks with no visible kernel in the causal range (never candidates: the
  // chunks reach every block below the local ones)
  if (srows) {
    const int tl = lane >> 5;
    const int tok = t0 + tl;
    if (tok < a.n_q) {
      const int b_p = (a.q_pos0 + tok) >> 6;
      float* row = srows + (size_t)tok * a.n_blk;
      for (int blk = nchunks * (SEL_CHUNK / 4) + (lane & 31); blk <= b_p; blk += 32)
        row[blk] = kNegInf;
    }
  }
  // S^shared past the swept chunks: kernels no token of the tile sees
  if constexpr (SHARED) {
    const int tok = t0 + (lane >> 5);
    if (tok < a.n_q) {
      float* row = a.S_sh + (((size_t)b * a.h_kv + g) * a.n_q + tok) * a.n_c1;
      for (int j = nchunks * SEL_CHUNK + (lane & 31); j < a.n_c1; j += 32) row[j] = 0.f;
    }
  }
  if constexpr (SELECT) {
    if (tid == 0) a.marks[tile_id] = 0;
#pragma unroll
    for (int tl = 0; tl < 2; ++tl) {
      const int tok = t0 + tl;
      const size_t row = ((size_t)b * a.h_kv + g) * a.n_q + min(tok, a.n_q - 1);
      topk_emit<2>(w.tk, w.tkbuf, tl, lane, a.k, a.q_pos0 + min(tok, a.n_q - 1), a.N_init,
                   a.N_local, a.budget, a.idx + row * a.budget, a.n_sel + row, tok < a.n_q);
    }
  }
}

// ---------------------------------------------------------------------------
// Split-K selection for few query tokens (decode).
// ---------------------------------------------------------------------------
constexpr int SPLIT_CK = 256;   // kernels per workgroup

struct SplitArgs {
  const uint16_t* Q;
  const uint16_t* Kc1;
  const uint16_t* Kc2;  // coarse keys (LSE approximation), else null
  float* S_cmp;
  float* S_sh;      // S^shared [batch][h_kv][n_q][n_c1], or null
  float* logits;    // [batch*n_q][h_kv][16][n_c1p]  (z*c, -inf when invisible)
  float2* part;     // [batch*n_q][h_kv][nch][16]    (chunk max, chunk sum)
  float2* part2;    // [batch*n_q][h_kv][nch2][16]   the same over the coarse kernels
  // fused top-k (select_blocks), row = (b*h_kv + g)*n_q + t: per-chunk
  // candidate lists ([rows][nch][kc], null when not fused) and the outputs
  uint64_t* cand;
  int32_t* idx;
  int32_t* n_sel;
  int k, N_init, N_local, budget, kc;
  int n_q, q_pos0, h_kv, n_c1, n_c1p, n_c2, n_blk, nch, nch2;
  int64_t c1_cap, c2_cap;
  float c;
  // varlen batches (null: every sequence has n_kv keys and its queries start
  // at q_pos0): sequence b holds seq_lens[b] keys, its queries are the last
  // n_q; n_c1, n_c2, nch, nch2 are then those of the longest, n_kv
  const int32_t* seq_lens;
  int n_kv;
  // kernels [app_begin, app_end) of every sequence are formed from K here
  // (the decode step's append, infv2_select_blocks_append) instead of read:
  // the logits sweep uses them and the workgroups of query token 0 write
  // them to Kc1_out.  K [b][kv_cap][h_kv][d]; app_end <= app_begin: none.
  const uint16_t* K;
  uint16_t* Kc1_out;
  int64_t kv_cap;
  int app_begin, app_end, l_C1, s_C1;
  double inv_l1;
};

// position of sequence b's first query token
__device__ __forceinline__ int split_pos0(const SplitArgs& a, int b) {
  return a.seq_lens ? seq_len_of(a.seq_lens, b, a.n_q, a.n_kv) - a.n_q : a.q_pos0;
}
// complete (coarse) kernels of sequence b
__device__ __forceinline__ int split_rows(const SplitArgs& a, int b, bool coarse) {
  if (!a.seq_lens) return coarse ? a.n_c2 : a.n_c1;
  const int last = seq_len_of(a.seq_lens, b, a.n_q, a.n_kv) - 1;
  return (coarse ? last_visible_coarse(last) : last_visible_kernel(last)) + 1;
}

// z = Q K^T (raw dot products) for the 64 key rows jw .. jw+63 of one wave:
// the rows are loaded with coalesced loads (lanes 16r..16r+15 read one
// 256-byte row), staged through the wave's LDS 32 rows at a time and read
// back XOR-swizzled as MFMA fragments, free of bank conflicts.  Rows past
// n_rows-1 are clamped to it (the caller masks them); with no row at all
// nothing is read.  C layout: acc[nt][i] is head 4*(lane>>4)+i, row
// jw + 16*nt + (lane&15).
// The rows of the decode step's append: where in K the sequence's keys of
// this group start (kcol: offset to the lane's two features 2 lane, 2 lane +
// 1), the row range, and where to write them (null: only use them).
struct SplitAppend {
  const uint16_t* kcol;
  size_t row_stride;
  uint16_t* out;           // K^C1 rows of this sequence and group, or null
  int begin, end, l_len, s_len;
  double inv_l;
};

__device__ __forceinline__ void split_logits_mfma(const uint16_t* keys, int n_rows, int jw,
                                                  const uint16_t* qrow_base, int lane,
                                                  uint8_t* kst, f32x4 (&acc)[4],
                                                  bool appending = false,
                                                  const SplitAppend app = {}) {
  u32x4 v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int j = min(jw + 4 * i + (lane >> 4), n_rows - 1);
    v[i] = n_rows > 0 ? *(const u32x4*)(keys + (size_t)j * SEL_D + 8 * (lane & 15))
                      : u32x4{0u, 0u, 0u, 0u};
  }

  // the wave's first appended kernel, formed while the rows above are in
  // flight (its keys' loads overlap theirs); any further one is formed below
  int j_app = -1;
  uint32_t w_app = 0u;
  if (appending) {
    const int jb = max(app.begin, jw), je = min(min(app.end, jw + 64), n_rows);
    if (jb < je) {
      j_app = jb;
      w_app = kmean_pair_bf16(app.kcol, app.row_stride, jb, app.l_len, app.s_len, app.inv_l);
    }
  }
  // A operand: Q rows = heads (lane & 15), k = d
  bf16x8 qf[4];
  const uint16_t* qrow = qrow_base + (size_t)(lane & 15) * SEL_D;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) qf[ks] = as_bf16x8(*(const u32x4*)(qrow + 32 * ks + 8 * (lane >> 4)));
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    // rows 32h .. 32h+31 of the wave's 64 (row 4i + (lane>>4) came from v[i])
#pragma unroll
    for (int i = 8 * h; i < 8 * h + 8; ++i) {
      const int row = 4 * i + (lane >> 4) - 32 * h, c16 = lane & 15;
      *(u32x4*)(kst + row * SEL_ROW_BYTES + ((c16 ^ (row & 15)) << 4)) = v[i];
    }
    // appended kernels of this half: formed from the keys (all 64 lanes, two
    // features each) in place of the rows just staged (not yet written in
    // memory), and written back by one query token's workgroups
    const int j_lo = jw + 32 * h;
    if (appending && j_lo < app.end && j_lo + 32 > app.begin) {
      const int r1 = min(min(app.end, j_lo + 32), n_rows);
      for (int j = max(app.begin, j_lo); j < r1; ++j) {
        const uint32_t w = j == j_app ? w_app
                                      : kmean_pair_bf16(app.kcol, app.row_stride, j, app.l_len,
                                                        app.s_len, app.inv_l);
        const int row = j - j_lo, c16 = lane >> 2;
        *(uint32_t*)(kst + row * SEL_ROW_BYTES + ((c16 ^ (row & 15)) << 4) + 4 * (lane & 3)) = w;
        if (app.out) *(uint32_t*)(app.out + (size_t)j * SEL_D + 2 * lane) = w;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int nt = 2 * h; nt < 2 * h + 2; ++nt) {
      acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int row = 16 * nt + (lane & 15) - 32 * h;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int c16 = 4 * ks + (lane >> 4);
        const bf16x8 kf = as_bf16x8(*(const u32x4*)(kst + row * SEL_ROW_BYTES + ((c16 ^ (row & 15)) << 4)));
        acc[nt] = mfma16(qf[ks], kf, acc[nt]);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

// Per-head (max, sum) of a workgroup's 256 masked logits zc (times c, -inf
// when not visible), acc as left by split_logits_mfma after scaling: mc =
// the chunk maximum, s = sum of 2^(zc - mc).  Every thread gets the values of
// the heads it holds (4*(lane>>4)+i).
__device__ __forceinline__ void split_chunk_partials(const f32x4 (&acc)[4], int lane, int wave,
                                                     float (&red_m)[4][16], float (&red_s)[4][16],
                                                     float (&mc_out)[4], float (&s_out)[4]) {
  float mloc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float m = kNegInf;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) m = fmaxf(m, acc[nt][i]);
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    mloc[i] = m;
  }
  if ((lane & 15) == 0)
#pragma unroll
    for (int i = 0; i < 4; ++i) red_m[wave][4 * (lane >> 4) + i] = mloc[i];
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = 4 * (lane >> 4) + i;
    const float mc = fmaxf(fmaxf(red_m[0][h], red_m[1][h]), fmaxf(red_m[2][h], red_m[3][h]));
    float s = 0.f;
    if (mc != kNegInf) {
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) s += fast_exp2(acc[nt][i] - mc);
    }
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) s += __shfl_xor(s, o, 64);
    if ((lane & 15) == 0) red_s[wave][h] = s;
    mc_out[i] = mc;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = 4 * (lane >> 4) + i;
    s_out[i] = red_s[0][h] + red_s[1][h] + red_s[2][h] + red_s[3][h];
  }
}

// grid: x = chunk, y = group, z = batch*n_q token.  4 waves x 64 kernels.
// Fine: writes z*c (-inf when not visible) to the logits buffer and the
// chunk's per-head (max, sum).  COARSE: the same sweep over the coarse
// kernels for the LSE approximation, partials only.
// APPEND: kernels [a.app_begin, a.app_end) are formed from K in the sweep
// (the decode step's append) -- a separate instance, so that the others keep
// their registers; held to 128 VGPRs (four waves per SIMD) so that its 1024
// workgroups fit the chip in one round, as the plain instance's do.
template <bool COARSE, bool APPEND = false>
__global__ void __launch_bounds__(256, APPEND ? 4 : 1) scores_split_logits_kernel(SplitArgs a) {
  __shared__ float red_m[4][16], red_s[4][16];
  __shared__ __attribute__((aligned(16))) uint8_t kst_all[4][32 * SEL_ROW_BYTES];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int chunk = blockIdx.x, g = blockIdx.y, bt = blockIdx.z;
  if constexpr (APPEND) {
    // chunks from the last one down, every row's before the next chunk: the
    // workgroups that form the appended kernels (the last chunks) start first
    const int rows = gridDim.y * gridDim.z;
    const int lin = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
    chunk = gridDim.x - 1 - lin / rows;
    const int r = lin % rows;
    g = r % gridDim.y;
    bt = r / gridDim.y;
  }
  const int b = bt / a.n_q, t = bt % a.n_q;
  const int p = split_pos0(a, b) + t;
  const int jmax = COARSE ? last_visible_coarse(p) : last_visible_kernel(p);
  const int hq = a.h_kv * SEL_G;
  const uint16_t* keys = COARSE ? a.Kc2 + ((size_t)b * a.h_kv + g) * a.c2_cap * SEL_D
                                : a.Kc1 + ((size_t)b * a.h_kv + g) * a.c1_cap * SEL_D;
  const int n_rows = split_rows(a, b, COARSE);
  const int jw = chunk * SPLIT_CK + wave * 64;
  f32x4 acc[4];
  SplitAppend app = {};
  const bool appending = APPEND && a.app_end > a.app_begin;
  if (appending) {
    app.kcol = a.K + ((size_t)b * a.kv_cap * a.h_kv + g) * SEL_D + 2 * lane;
    app.row_stride = (size_t)a.h_kv * SEL_D;
    app.out = t == 0 ? a.Kc1_out + ((size_t)b * a.h_kv + g) * a.c1_cap * SEL_D : nullptr;
    app.begin = a.app_begin;
    app.end = a.app_end;
    app.l_len = a.l_C1;
    app.s_len = a.s_C1;
    app.inv_l = a.inv_l1;
  }
  split_logits_mfma(keys, n_rows, jw, a.Q + (((size_t)b * a.n_q + t) * hq + g * SEL_G) * SEL_D,
                    lane, kst_all[wave], acc, appending, app);
  float* lrow = a.logits + ((size_t)bt * a.h_kv + g) * SEL_G * a.n_c1p;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = 4 * (lane >> 4) + i;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int j = jw + 16 * nt + (lane & 15);
      const float zc = (j <= jmax) ? acc[nt][i] * a.c : kNegInf;
      acc[nt][i] = zc;
      if (!COARSE && j < a.n_c1p) lrow[(size_t)h * a.n_c1p + j] = zc;
    }
  }
  float mc[4], sc[4];
  split_chunk_partials(acc, lane, wave, red_m, red_s, mc, sc);
  if (wave == 0 && (lane & 15) == 0) {
    float2* part = COARSE ? a.part2 + (((size_t)bt * a.h_kv + g) * a.nch2 + chunk) * SEL_G
                          : a.part + (((size_t)bt * a.h_kv + g) * a.nch + chunk) * SEL_G;
#pragma unroll
    for (int i = 0; i < 4; ++i) part[4 * (lane >> 4) + i] = make_float2(mc[i], sc[i]);
  }
}

// Each head's softmax reference and sum from per-chunk (max, sum) partials
// [.][nch][16] of a row: threads 0..255, 16 per head, each folding every
// 16th chunk, then a 16-lane merge; thread 16h returns head h's (m, s).
// Every product-sum is an explicit fma, so all kernels that call this round
// identically.
__device__ __forceinline__ float2 head_lse_merge(const float2* part, int nch, int h_kv, int g,
                                                 int bt, int tid) {
  const int h = tid >> 4, q = tid & 15;
  const float2* pr = part + ((size_t)bt * h_kv + g) * nch * SEL_G + h;
  float m = kNegInf, s = 0.f;
  for (int c = q; c < nch; c += 16) {
    const float2 v = pr[(size_t)c * SEL_G];
    if (v.x == kNegInf) continue;
    if (v.x > m) { s = __builtin_fmaf(s, fast_exp2(m - v.x), v.y); m = v.x; }
    else s = __builtin_fmaf(v.y, fast_exp2(v.x - m), s);
  }
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) {
    const float mo = __shfl_xor(m, o, 64), so = __shfl_xor(s, o, 64);
    const float mn = fmaxf(m, mo);
    if (mn != kNegInf) {
      const float e = __builtin_fmaf(s, fast_exp2(m - mn), 0.f);
      s = __builtin_fmaf(so, fast_exp2(mo - mn), e);
    }
    m = mn;
  }
  return make_float2(m, s);
}

// Mh[h] = the running maximum (0 when nothing is visible), Wh[h] = 1 / sum of
// exp2(z - Mh[h]) over the row's fine kernels.
__device__ __forceinline__ void head_lse_weights(const SplitArgs& a, int g, int bt, int tid,
                                                 float* Mh, float* Wh) {
  const float2 ms = head_lse_merge(a.part, a.nch, a.h_kv, g, bt, tid);
  if ((tid & 15) == 0) {
    const int h = tid >> 4;
    Mh[h] = (ms.x == kNegInf) ? 0.f : ms.x;
    Wh[h] = ms.y > 0.f ? 1.0f / ms.y : 0.f;
  }
}

// S^shared of the chunk's kernels j0 .. j0+255 from sh (sh[x] = kernel
// j0 - 1 + x, -inf where not visible) into the caller's row: 0 where the
// token does not see the kernel.  256 threads, one kernel each.
static_assert(SPLIT_CK == 256, "one thread per kernel of the chunk");
__device__ __forceinline__ void split_write_shared(const SplitArgs& a, int b, int g, int t,
                                                   int j0, const float* sh) {
  const int j = j0 + (int)threadIdx.x;
  if (j < a.n_c1) {
    const float v = sh[1 + threadIdx.x];
    a.S_sh[(((size_t)b * a.h_kv + g) * a.n_q + t) * a.n_c1 + j] = (v == kNegInf) ? 0.f : v;
  }
}

// The pool step for one chunk: merges the per-chunk (max, sum) partials of
// every head into the exact log-sum-exp, forms S^shared for the chunk's 256
// kernels (+ the carry kernel) and max-pools them into its 64 blocks; thread
// bb < 64 returns block chunk*64 + bb's score (-inf when not causal).  S^cmp
// is written when S_cmp is not null.  256 threads.
__device__ __forceinline__ float split_pool_chunk(const SplitArgs& a, int chunk, int g, int bt,
                                                  float* Mh, float* Wh, float* sh) {
  const int b = bt / a.n_q, t = bt % a.n_q;
  const int p = split_pos0(a, b) + t;
  const int jmax = last_visible_kernel(p);
  const int b_p = p >> 6;
  head_lse_weights(a, g, bt, threadIdx.x, Mh, Wh);
  __syncthreads();
  const float* lrow = a.logits + ((size_t)bt * a.h_kv + g) * SEL_G * a.n_c1p;
  const int j0 = chunk * SPLIT_CK;
  for (int x = threadIdx.x; x <= SPLIT_CK; x += blockDim.x) {
    const int j = j0 - 1 + x;       // x = 0 is the carry kernel j0-1
    float v = kNegInf;
    if (j >= 0 && j <= jmax) {
      v = 0.f;
#pragma unroll
      for (int h = 0; h < SEL_G; ++h)
        v = __builtin_fmaf(fast_exp2(lrow[(size_t)h * a.n_c1p + j] - Mh[h]), Wh[h], v);
    }
    sh[x] = v;
  }
  __syncthreads();
  if (a.S_sh) split_write_shared(a, b, g, t, j0, sh);
  float* row = a.S_cmp ? a.S_cmp + (((size_t)b * a.h_kv + g) * a.n_q + t) * a.n_blk : nullptr;
  const int nblk_chunk = SPLIT_CK / 4;
  float out = kNegInf;
  if (threadIdx.x < nblk_chunk) {
    const int bb = threadIdx.x;
    const int blk = chunk * nblk_chunk + bb;
    float v = sh[4 * bb];
#pragma unroll
    for (int q = 1; q < 5; ++q) v = fmaxf(v, sh[4 * bb + q]);
    if (row && blk <= b_p) row[blk] = v;
    out = v;
  }
  if (row && chunk == a.nch - 1)
    for (int blk = a.nch * nblk_chunk + threadIdx.x; blk <= b_p; blk += blockDim.x)
      row[blk] = kNegInf;
  return out;
}

// grid as above; 256 threads = 256 kernels of the chunk (+ the carry kernel).
// With the top-k fused in (a.cand set), wave 0 also writes the chunk's kc
// best candidate blocks, sorted, as 64-bit keys: order-preserving score bits
// << 32 | ~blk, unique, and at equal scores the lower block ranks higher;
// 0 marks "no candidate".
__global__ void __launch_bounds__(256) scores_split_pool_kernel(SplitArgs a) {
  __shared__ float Mh[SEL_G], Wh[SEL_G];
  __shared__ float sh[SPLIT_CK + 1];
  const int chunk = blockIdx.x, g = blockIdx.y, bt = blockIdx.z;
  const float v = split_pool_chunk(a, chunk, g, bt, Mh, Wh, sh);
  if (a.cand == nullptr || threadIdx.x >= 64) return;     // whole waves leave
  const int lane = threadIdx.x;
  const int b = bt / a.n_q, t = bt % a.n_q;
  const int b_p = (split_pos0(a, b) + t) >> 6;
  const int init_hi = min(a.N_init, b_p + 1);
  const int loc_lo = max(0, b_p - a.N_local + 1);
  const int blk = chunk * 64 + lane;
  const bool cand = blk >= init_hi && blk < loc_lo;
  const uint64_t key = cand ? ((uint64_t)ordered_bits(v) << 32) | (uint64_t)(~(uint32_t)blk) : 0ull;
  const uint64_t sorted = wave_sort_desc<uint64_t>(key, lane);
  const size_t row = ((size_t)b * a.h_kv + g) * a.n_q + t;
  if (lane < a.kc) a.cand[(row * a.nch + chunk) * a.kc + lane] = sorted;
}

// The LSE approximation for few query tokens, in one sweep over K^C1: a
// workgroup takes 256 kernels of a row (grid as the logits kernel), takes
// each head's log2-normaliser L[h] from the coarse partials (a token that
// sees no coarse kernel has all its visible kernels in chunk 0, whose
// workgroup takes the exact LSE from its own logits), forms
// S^shared = sum_h 2^(z*c - L[h]) for its kernels and the kernel before them
// (a plain dot product), max-pools its 64 blocks and writes S^cmp (when
// S_cmp is set) and, with LISTS, the chunk's sorted candidate list as the
// pool kernel does.
template <bool LISTS>
__global__ void __launch_bounds__(256) scores_split_fused_kernel(SplitArgs a) {
  __shared__ float red_m[4][16], red_s[4][16];
  __shared__ __attribute__((aligned(16))) uint8_t kst_all[4][32 * SEL_ROW_BYTES];
  __shared__ float Lh[SEL_G];
  __shared__ float sh[SPLIT_CK + 1];    // sh[x] = S^shared of kernel j0 - 1 + x
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int chunk = blockIdx.x, g = blockIdx.y, bt = blockIdx.z;
  const int b = bt / a.n_q, t = bt % a.n_q;
  const int p = split_pos0(a, b) + t;
  const int jmax = last_visible_kernel(p);
  const bool coarse = last_visible_coarse(p) >= 0;      // row-uniform
  const int hq = a.h_kv * SEL_G;
  const int j0 = chunk * SPLIT_CK;
  const uint16_t* qbase = a.Q + (((size_t)b * a.n_q + t) * hq + g * SEL_G) * SEL_D;
  const uint16_t* kc1 = a.Kc1 + ((size_t)b * a.h_kv + g) * a.c1_cap * SEL_D;
  if (coarse) {
    // L = M + log2(s) + log2(s_C2/s_C1) from the coarse partials
    const float2 ms = head_lse_merge(a.part2, a.nch2, a.h_kv, g, bt, tid);
    if ((tid & 15) == 0) Lh[tid >> 4] = ms.x + (fast_log2(ms.y) + kLog2CoarseRatio);
  }
  const int jw = j0 + wave * 64;
  f32x4 acc[4];
  split_logits_mfma(kc1, split_rows(a, b, false), jw, qbase, lane, kst_all[wave], acc);
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int j = jw + 16 * nt + (lane & 15);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[nt][i] = (j <= jmax) ? acc[nt][i] * a.c : kNegInf;
  }
  if (!coarse) {
    // no coarse kernel: the exact LSE (every visible kernel is in chunk 0;
    // later chunks see none and only write -inf)
    float mc[4], sc[4];
    split_chunk_partials(acc, lane, wave, red_m, red_s, mc, sc);
    if (wave == 0 && (lane & 15) == 0)
#pragma unroll
      for (int i = 0; i < 4; ++i) Lh[4 * (lane >> 4) + i] = mc[i] + fast_log2(sc[i]);
  }
  // the kernel before the chunk (block 64*chunk takes kernels j0-1 .. j0+3):
  // wave 3, lane = 4 * head + quarter of d
  float carry_part = 0.f;
  const int jc = j0 - 1;
  const bool carry_vis = chunk > 0 && jc <= jmax;
  if (wave == 3 && carry_vis) {
    const int h = lane >> 2, qd = lane & 3;
    const uint16_t* qrow = qbase + (size_t)h * SEL_D + 32 * qd;
    const uint16_t* krow = kc1 + (size_t)jc * SEL_D + 32 * qd;
    float z = 0.f;
#pragma unroll
    for (int e = 0; e < 32; e += 8) {
      const u32x4 qv = *(const u32x4*)(qrow + e), kv = *(const u32x4*)(krow + e);
      const uint32_t qw[4] = {qv[0], qv[1], qv[2], qv[3]}, kw[4] = {kv[0], kv[1], kv[2], kv[3]};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        z = __builtin_fmaf(__uint_as_float(qw[u] << 16), __uint_as_float(kw[u] << 16), z);
        z = __builtin_fmaf(__uint_as_float(qw[u] & 0xFFFF0000u), __uint_as_float(kw[u] & 0xFFFF0000u), z);
      }
    }
    z += __shfl_xor(z, 1, 64);
    z += __shfl_xor(z, 2, 64);
    carry_part = z;   // every lane of the head's quad holds the dot product
  }
  __syncthreads();    // Lh ready
  // S^shared of the wave's 64 kernels: the lane's 4 heads, then the 4 lane rows
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    float v = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) v += fast_exp2(acc[nt][i] - Lh[4 * (lane >> 4) + i]);
    v += __shfl_xor(v, 16, 64);
    v += __shfl_xor(v, 32, 64);
    const int j = jw + 16 * nt + (lane & 15);
    if ((lane >> 4) == nt) sh[1 + wave * 64 + 16 * nt + (lane & 15)] = (j <= jmax) ? v : kNegInf;
  }
  if (wave == 3) {
    float v = 0.f;
    if (carry_vis) {
      v = (lane & 3) == 0 ? fast_exp2(__builtin_fmaf(carry_part, a.c, -Lh[lane >> 2])) : 0.f;
#pragma unroll
      for (int o = 4; o < 64; o <<= 1) v += __shfl_xor(v, o, 64);
    }
    if (lane == 0) sh[0] = carry_vis ? v : kNegInf;
  }
  __syncthreads();
  if (a.S_sh) split_write_shared(a, b, g, t, j0, sh);
  const int b_p = p >> 6;
  float* srow = a.S_cmp ? a.S_cmp + (((size_t)b * a.h_kv + g) * a.n_q + t) * a.n_blk : nullptr;
  if (srow && chunk == a.nch - 1)
    for (int blk = a.nch * 64 + tid; blk <= b_p; blk += 256) srow[blk] = kNegInf;
  if (wave != 0) return;
  const int blk = chunk * 64 + lane;
  float v = sh[4 * lane];
#pragma unroll
  for (int q = 1; q < 5; ++q) v = fmaxf(v, sh[4 * lane + q]);
  if (srow && blk <= b_p) srow[blk] = v;
  if constexpr (LISTS) {
    const int init_hi = min(a.N_init, b_p + 1);
    const int loc_lo = max(0, b_p - a.N_local + 1);
    const bool cand = blk >= init_hi && blk < loc_lo;
    const uint64_t key = cand ? ((uint64_t)ordered_bits(v) << 32) | (uint64_t)(~(uint32_t)blk) : 0ull;
    const uint64_t sorted = wave_sort_desc<uint64_t>(key, lane);
    const size_t row = ((size_t)b * a.h_kv + g) * a.n_q + t;
    if (lane < a.kc) a.cand[(row * a.nch + chunk) * a.kc + lane] = sorted;
  }
}

// The top-k of the fused selection, one workgroup per row (token, group),
// from the sorted per-chunk candidate lists of the pool kernel:
//   * the kk-th best key K* is bounded from below by the kk-th best of the
//     first r = ceil(kk / nch) keys of every list (those nch*r >= kk keys are
//     distinct, so at least kk keys reach the bound); the keys at or above the
//     bound (usually a few more than kk) are sorted by one wave;
//   * the selection is init/local plus the candidates with key >= K*, written
//     in ascending block order with -1 padding.
constexpr int MERGE_THREADS = 256;
constexpr int MERGE_WAVES = MERGE_THREADS / 64;
constexpr int SELECT_MAX_CHUNKS = 64;      // rows of up to 64 * 256 kernels
constexpr int SELECT_MAX_KC = 32;          // k <= 32
constexpr int SELECT_MAX_KEYS = 1024;      // chunks * k <= 1024
__global__ void __launch_bounds__(MERGE_THREADS) scores_select_merge_kernel(SplitArgs a) {
  __shared__ uint64_t keys[SELECT_MAX_KEYS];
  __shared__ uint64_t pick[64];
  __shared__ uint32_t selbits[SELECT_MAX_CHUNKS * 2 + 2];   // blocks 0 .. 64 * nch
  __shared__ uint32_t count_s;
  __shared__ uint64_t kstar_s, bound_s;
  __shared__ int wave_cnt[MERGE_WAVES];
  const int g = blockIdx.x, bt = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = bt / a.n_q, t = bt % a.n_q;
  const size_t row = ((size_t)b * a.h_kv + g) * a.n_q + t;
  const int b_p = (split_pos0(a, b) + t) >> 6;
  const int nb = b_p + 1;
  const int init_hi = min(a.N_init, nb);
  const int loc_lo = max(0, b_p - a.N_local + 1);
  const int ncand = max(0, loc_lo - init_hi);
  const int kk = min(a.k, ncand);
  // only the chunks that hold candidate blocks (< loc_lo) have non-zero keys:
  // the bound and the scans below use those lists alone
  const int nch = ncand > 0 ? min(a.nch, (loc_lo + 63) >> 6) : 1;
  const int nkeys = nch * a.kc;
  const uint64_t* rlist = a.cand + row * (size_t)(a.nch * a.kc);
  for (int i = tid; i < nkeys; i += MERGE_THREADS) keys[i] = rlist[i];
  for (int i = tid; i < SELECT_MAX_CHUNKS * 2 + 2; i += MERGE_THREADS) selbits[i] = 0u;
  if (tid < 64) pick[tid] = 0ull;
  if (tid == 0) count_s = 0u;
  __syncthreads();
  uint64_t kstar = 1ull;   // keys >= kstar are selected; every candidate key is >= 1
  if (kk > 0 && kk < ncand) {
    const int r = (kk + nch - 1) / nch;   // nch * r <= 64 as kk <= 32, nch <= 64
    if (wave == 0) {
      const uint64_t e = lane < nch * r ? keys[(lane / r) * a.kc + lane % r] : 0ull;
      const uint64_t sorted = wave_sort_desc<uint64_t>(e, lane);
      if (lane == kk - 1) bound_s = sorted > 1ull ? sorted : 1ull;
    }
    __syncthreads();
    const uint64_t bound = bound_s;
    for (int i = tid; i < nkeys; i += MERGE_THREADS) {
      const uint64_t kv = keys[i];
      if (kv >= bound) {
        const uint32_t pos = atomicAdd(&count_s, 1u);
        if (pos < 64) pick[pos] = kv;
      }
    }
    __syncthreads();
    if (count_s <= 64) {
      if (wave == 0) {
        const uint64_t sorted = wave_sort_desc<uint64_t>(pick[lane], lane);
        if (lane == kk - 1) kstar_s = sorted;
      }
    } else {
      // many keys at or above the bound: rank each against every key
      for (int i = tid; i < nkeys; i += MERGE_THREADS) {
        const uint64_t kv = keys[i];
        if (kv < bound) continue;
        int above = 0;
        for (int j = 0; j < nkeys; ++j) above += keys[j] > kv ? 1 : 0;
        if (above == kk - 1) kstar_s = kv;
      }
    }
    __syncthreads();
    kstar = kstar_s;
  }
  // selection bitmap: init/local blocks and the candidates with key >= K*
  for (int blk = tid; blk < nb; blk += MERGE_THREADS)
    if (blk < init_hi || blk >= loc_lo) atomicOr(&selbits[blk >> 5], 1u << (blk & 31));
  if (kk > 0)
    for (int i = tid; i < nkeys; i += MERGE_THREADS) {
      const uint64_t kv = keys[i];
      if (kv != 0ull && kv >= kstar) {
        const uint32_t blk = ~(uint32_t)kv;
        atomicOr(&selbits[blk >> 5], 1u << (blk & 31));
      }
    }
  __syncthreads();
  // ascending compaction: thread i takes bitmap word i (blocks 32i..32i+31)
  const int nwords = (nb + 31) >> 5;
  const uint32_t word = tid < nwords ? selbits[tid] : 0u;
  const int cnt = __popc(word);
  int incl = cnt;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  if (lane == 63) wave_cnt[wave] = incl;
  __syncthreads();
  int base = 0, total = 0;
#pragma unroll
  for (int w = 0; w < MERGE_WAVES; ++w) {
    base += w < wave ? wave_cnt[w] : 0;
    total += wave_cnt[w];
  }
  int pos = base + incl - cnt;
  int32_t* out = a.idx + row * a.budget;
  for (uint32_t wv = word; wv; wv &= wv - 1) out[pos++] = tid * 32 + __builtin_ctz(wv);
  for (int i = total + tid; i < a.budget; i += MERGE_THREADS) out[i] = -1;
  if (tid == 0) a.n_sel[row] = total;
}

// ---------------------------------------------------------------------------
// Generic selection: any G, d, B, l_C1, s_C1 and fp32 or bf16 I/O; fp64 math.
// One workgroup per (token, group).  Dynamic LDS: (n_vis + 1) doubles + G
// doubles.
// ---------------------------------------------------------------------------
struct GenericScoresArgs {
  const void* Q;
  const void* Kc1;
  const void* Kc2;   // coarse keys (LSE approximation), else null
  float* S_cmp;
  float* S_sh;       // S^shared [batch][h_kv][n_q][n_c1], or null
  int dtype, n_q, q_pos0, h_kv, G, d, n_c1, n_c2, n_blk, B, l_C1, s_C1;
  int approx;
  int64_t c1_cap, c2_cap;
  double scale;
};

template <typename T> __device__ __forceinline__ double ld(const T* p, size_t i);
template <> __device__ __forceinline__ double ld<float>(const float* p, size_t i) { return p[i]; }
template <> __device__ __forceinline__ double ld<uint16_t>(const uint16_t* p, size_t i) {
  return (double)bf16_bits_to_f32(p[i]);
}

__device__ double block_reduce_max(double v, double* red) {
  for (int o = 32; o > 0; o >>= 1) v = fmax(v, __shfl_xor(v, o, 64));
  const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  double r = red[0];
  for (int i = 1; i < nw; ++i) r = fmax(r, red[i]);
  return r;
}
__device__ double block_reduce_sum(double v, double* red) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  double r = 0.0;
  for (int i = 0; i < nw; ++i) r += red[i];
  return r;
}

template <typename T>
__global__ void __launch_bounds__(256) scores_generic_kernel(GenericScoresArgs a) {
  extern __shared__ double dyn[];
  __shared__ double red[8];
  const int t = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int p = a.q_pos0 + t;
  const int jmax = p >= a.l_C1 - 1 ? (p - a.l_C1 + 1) / a.s_C1 : -1;
  const int nv = min(jmax + 1, a.n_c1);
  double* lse = dyn;            // [G]
  double* shared_s = dyn + a.G; // [nv]
  const T* Q = (const T*)a.Q;
  const T* K = (const T*)a.Kc1;
  const int hq = a.h_kv * a.G;
  const T* kbase = K + ((size_t)b * a.h_kv + g) * a.c1_cap * a.d;
  // LSE approximation: coarse kernels of length 4 l_C1 and stride 4 s_C1
  const int l2 = 4 * a.l_C1, s2 = 4 * a.s_C1;
  const int nv2 = a.approx ? min(p >= l2 - 1 ? (p - l2 + 1) / s2 + 1 : 0, a.n_c2) : 0;
  const T* k2base = nv2 > 0 ? (const T*)a.Kc2 + ((size_t)b * a.h_kv + g) * a.c2_cap * a.d : nullptr;
  for (int h = 0; h < a.G; ++h) {
    const T* q = Q + (((size_t)b * a.n_q + t) * hq + g * a.G + h) * a.d;
    if (nv2 > 0) {
      // lse~ = log sum over the visible coarse kernels of exp(z2) + ln(s_C2/s_C1)
      double m = -__builtin_huge_val();
      for (int j = threadIdx.x; j < nv2; j += blockDim.x) {
        double z = 0.0;
        for (int i = 0; i < a.d; ++i) z += ld<T>(q, i) * ld<T>(k2base, (size_t)j * a.d + i);
        m = fmax(m, z * a.scale);
      }
      m = block_reduce_max(m, red);
      double s = 0.0;
      for (int j = threadIdx.x; j < nv2; j += blockDim.x) {
        double z = 0.0;
        for (int i = 0; i < a.d; ++i) z += ld<T>(q, i) * ld<T>(k2base, (size_t)j * a.d + i);
        s += exp(z * a.scale - m);
      }
      s = block_reduce_sum(s, red);
      if (threadIdx.x == 0) lse[h] = m + log(s) + log((double)s2 / (double)a.s_C1);
      continue;
    }
    double m = -__builtin_huge_val();
    for (int j = threadIdx.x; j < nv; j += blockDim.x) {
      double z = 0.0;
      for (int i = 0; i < a.d; ++i) z += ld<T>(q, i) * ld<T>(kbase, (size_t)j * a.d + i);
      m = fmax(m, z * a.scale);
    }
    m = block_reduce_max(m, red);
    double s = 0.0;
    for (int j = threadIdx.x; j < nv; j += blockDim.x) {
      double z = 0.0;
      for (int i = 0; i < a.d; ++i) z += ld<T>(q, i) * ld<T>(kbase, (size_t)j * a.d + i);
      s += exp(z * a.scale - m);
    }
    s = block_reduce_sum(s, red);
    if (threadIdx.x == 0) lse[h] = nv > 0 ? m + log(s) : -__builtin_huge_val();
  }
  __syncthreads();
  for (int j = threadIdx.x; j < nv; j += blockDim.x) {
    double acc = 0.0;
    for (int h = 0; h < a.G; ++h) {
      const T* q = Q + (((size_t)b * a.n_q + t) * hq + g * a.G + h) * a.d;
      double z = 0.0;
      for (int i = 0; i < a.d; ++i) z += ld<T>(q, i) * ld<T>(kbase, (size_t)j * a.d + i);
      acc += exp(z * a.scale - lse[h]);
    }
    shared_s[j] = acc;
  }
  __syncthreads();
  if (a.S_sh) {   // 0 for the kernels the token does not see
    float* srow = a.S_sh + (((size_t)b * a.h_kv + g) * a.n_q + t) * a.n_c1;
    for (int j = threadIdx.x; j < a.n_c1; j += blockDim.x) srow[j] = j < nv ? (float)shared_s[j] : 0.f;
  }
  const int b_p = p / a.B;
  float* row = a.S_cmp + (((size_t)b * a.h_kv + g) * a.n_q + t) * a.n_blk;
  for (int blk = threadIdx.x; blk <= b_p; blk += blockDim.x) {
    // kernels whose span [j*s_C1, j*s_C1+l_C1-1] meets [blk*B, blk*B+B-1]
    const int lo_num = blk * a.B - a.l_C1 + 1;
    int jlo = lo_num <= 0 ? 0 : (lo_num + a.s_C1 - 1) / a.s_C1;
    int jhi = (blk * a.B + a.B - 1) / a.s_C1;
    if (jhi > nv - 1) jhi = nv - 1;
    double v = -__builtin_huge_val();
    for (int j = jlo; j <= jhi; ++j) v = fmax(v, shared_s[j]);
    row[blk] = (float)v;
  }
}

// ---------------------------------------------------------------------------
bool scores_fast_shape(const infv2_problem& p) {
  return p.dtype == INFV2_BF16 && p.G == SEL_G && p.d == SEL_D && p.B == 64 && p.l_C1 == 32 &&
         p.s_C1 == 16;
}
bool scores_use_split(const infv2_problem& p) { return scores_fast_shape(p) && p.n_q <= 4; }

static int split_nch(int n_c1) { return (n_c1 + 1 + SPLIT_CK - 1) / SPLIT_CK; }
static int split_nch2(int n_c2) { return (n_c2 + SPLIT_CK - 1) / SPLIT_CK; }
static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Split path workspace: exact LSE: the logits and the fine partials; LSE
// approximation: the coarse partials only (one sweep, no logits).
size_t scores_workspace(const infv2_problem& p, const KeySet& ks) {
  if (!scores_use_split(p)) return 0;
  const size_t rows = (size_t)p.batch * p.n_q * p.h_kv;
  if (p.lse_approx) return rows * split_nch2(ks.n_c2) * SEL_G * sizeof(float2);
  const int n_c1p = (ks.n_c1 + 63) & ~63;
  return rows * SEL_G * (size_t)n_c1p * sizeof(float) +
         rows * split_nch(ks.n_c1) * SEL_G * sizeof(float2);
}

size_t scores_generic_lds(const infv2_problem& p, int n_c1) {
  return (size_t)(n_c1 + p.G + 1) * sizeof(double);
}

static SplitArgs split_args(const infv2_problem& p, const void* Q, const KeySet& ks,
                            float* S_cmp, void* ws, int n_blk, float scale) {
  SplitArgs a = {};
  a.Q = (const uint16_t*)Q;
  a.Kc1 = (const uint16_t*)ks.Kc1;
  a.Kc2 = (const uint16_t*)ks.Kc2;
  a.S_cmp = S_cmp;
  a.n_q = p.n_q;
  a.q_pos0 = p.q_pos0;
  a.h_kv = p.h_kv;
  a.n_c1 = ks.n_c1;
  a.n_c1p = (ks.n_c1 + 63) & ~63;
  a.n_c2 = ks.n_c2;
  a.n_blk = n_blk;
  a.nch = split_nch(ks.n_c1);
  a.nch2 = split_nch2(ks.n_c2);
  a.c1_cap = ks.c1_cap;
  a.c2_cap = ks.c2_cap;
  a.c = scale * kLog2e;
  const size_t rows = (size_t)p.batch * p.n_q * p.h_kv;
  if (p.lse_approx) {
    a.part2 = (float2*)ws;
  } else {
    a.logits = (float*)ws;
    a.part = (float2*)((char*)ws + rows * SEL_G * (size_t)a.n_c1p * sizeof(float));
  }
  return a;
}

// The selection scores of the split path: exact LSE: logits (fine partials)
// then pool; approximation: coarse partials, then one fused sweep over K^C1.
// With a.cand set the pool / fused kernel also writes the candidate lists.
static void launch_split_scores(const infv2_problem& p, const SplitArgs& a, hipStream_t stream) {
  const dim3 grid(a.nch, p.h_kv, p.batch * p.n_q);
  if (p.lse_approx) {
    if (a.nch2 > 0)
      hipLaunchKernelGGL(scores_split_logits_kernel<true>, dim3(a.nch2, p.h_kv, p.batch * p.n_q),
                         dim3(256), 0, stream, a);
    if (a.cand)
      hipLaunchKernelGGL(scores_split_fused_kernel<true>, grid, dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL(scores_split_fused_kernel<false>, grid, dim3(256), 0, stream, a);
  } else {
    if (a.app_end > a.app_begin)
      hipLaunchKernelGGL((scores_split_logits_kernel<false, true>), grid, dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL(scores_split_logits_kernel<false>, grid, dim3(256), 0, stream, a);
    hipLaunchKernelGGL(scores_split_pool_kernel, grid, dim3(256), 0, stream, a);
  }
}

static ScoresArgs prefill_args(const infv2_problem& p, const void* Q, const KeySet& ks,
                               float* S_cmp, int n_blk, float scale) {
  ScoresArgs a = {};
  a.Q = (const uint16_t*)Q;
  a.Kc1 = (const uint16_t*)ks.Kc1;
  a.Kc2 = (const uint16_t*)ks.Kc2;
  a.S_cmp = S_cmp;
  a.batch = p.batch;
  a.n_q = p.n_q;
  a.q_pos0 = p.q_pos0;
  a.h_kv = p.h_kv;
  a.n_c1 = ks.n_c1;
  a.n_c2 = ks.n_c2;
  a.n_blk = n_blk;
  a.tiles = (p.n_q + SEL_TOK_WG - 1) / SEL_TOK_WG;
  a.c1_cap = ks.c1_cap;
  a.c2_cap = ks.c2_cap;
  a.c = scale * kLog2e;
  return a;
}

// a.S_sh (S^shared wanted) takes the SHARED instance of the fast kernel; the
// selection mode never writes S^shared.
template <bool SELECT>
static void launch_prefill_scores(const infv2_problem& p, const ScoresArgs& a,
                                  hipStream_t stream) {
  const int wgs = a.tiles * p.h_kv * p.batch;
  dim3 grid(8 % p.h_kv == 0 ? ((wgs + 7) / 8) * 8 : wgs);
  const dim3 block(64 * FAST_WAVES);
  if (p.lse_approx) {
    if (!SELECT && a.S_sh)
      hipLaunchKernelGGL((scores_prefill_kernel<true, false, true>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((scores_prefill_kernel<true, SELECT>), grid, block, 0, stream, a);
    hipLaunchKernelGGL((scores_exact_kernel<true, SELECT>), dim3(wgs), dim3(256), 0, stream, a);
  } else {
    if (!SELECT && a.S_sh)
      hipLaunchKernelGGL((scores_prefill_kernel<false, false, true>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((scores_prefill_kernel<false, SELECT>), grid, block, 0, stream, a);
    hipLaunchKernelGGL((scores_exact_kernel<false, SELECT>), dim3(wgs), dim3(256), 0, stream, a);
  }
}

// The fused selection serves the split shapes (candidate lists from the pool
// kernel, then a per-row merge; at most 1024 candidate keys per row) and the
// fast prefill shapes (a streaming top-k inside the score sweep), with
// k <= 32 and a budget of at most 64 blocks.
bool select_fused_shape(const infv2_problem& p, int n_c1) {
  if (p.k > SELECT_MAX_KC || p.N_init + p.N_local + p.k > 64) return false;
  if (scores_use_split(p)) {
    const int nch = split_nch(n_c1);
    return nch <= SELECT_MAX_CHUNKS && nch * p.k <= SELECT_MAX_KEYS;
  }
  return scores_fast_shape(p);
}

// workspace beyond scores_workspace() rounded up to 256 bytes: the candidate
// lists (split shapes) or one mark per tile (prefill shapes)
size_t select_fused_workspace(const infv2_problem& p, int n_c1) {
  if (scores_use_split(p))
    return (size_t)p.batch * p.n_q * p.h_kv * split_nch(n_c1) * p.k * sizeof(uint64_t);
  return (size_t)p.batch * p.h_kv * ((p.n_q + SEL_TOK_WG - 1) / SEL_TOK_WG) * sizeof(int32_t);
}

// The split path of the fused selection: score sweeps that also write the
// per-chunk candidate lists, then the per-row merge.  seq_lens: varlen batch
// (the sizes in p and ks are then those of the longest sequence, n_kv).
static hipError_t launch_select_split(const infv2_problem& p, const void* Q, const KeySet& ks,
                                      const int32_t* seq_lens, float* S_cmp, int32_t* idx,
                                      int32_t* n_sel, void* ws, int n_blk, float scale,
                                      int budget, hipStream_t stream,
                                      const SplitArgs* append = nullptr,
                                      CandLists* lists_only = nullptr) {
  SplitArgs a = split_args(p, Q, ks, S_cmp, ws, n_blk, scale);
  if (append) {
    a.K = append->K;
    a.Kc1_out = append->Kc1_out;
    a.kv_cap = append->kv_cap;
    a.app_begin = append->app_begin;
    a.app_end = append->app_end;
    a.l_C1 = append->l_C1;
    a.s_C1 = append->s_C1;
    a.inv_l1 = append->inv_l1;
  }
  a.seq_lens = seq_lens;
  a.n_kv = p.n_kv;
  a.cand = (uint64_t*)((char*)ws + align256(scores_workspace(p, ks)));
  a.idx = idx;
  a.n_sel = n_sel;
  a.k = p.k;
  a.kc = p.k;
  a.N_init = p.N_init;
  a.N_local = p.N_local;
  a.budget = budget;
  launch_split_scores(p, a, stream);
  if (lists_only) {
    // the caller merges the lists itself (attn_split_select_kernel)
    lists_only->cand = a.cand;
    lists_only->nch = a.nch;
    lists_only->kc = a.kc;
    return hipGetLastError();
  }
  hipLaunchKernelGGL(scores_select_merge_kernel, dim3(p.h_kv, p.batch * p.n_q),
                     dim3(MERGE_THREADS), 0, stream, a);
  return hipGetLastError();
}

// Varlen batches (decode): the split selection with per-sequence lengths;
// requires scores_use_split(p) and select_fused_shape(p, n_C1(n_kv)).
hipError_t launch_select_varlen(const infv2_problem& p, const void* Q, const KeySet& ks,
                                const int32_t* seq_lens, int32_t* idx, int32_t* n_sel, void* ws,
                                int n_blk, float scale, int budget, hipStream_t stream) {
  return launch_select_split(p, Q, ks, seq_lens, nullptr, idx, n_sel, ws, n_blk, scale, budget,
                             stream);
}

hipError_t launch_select_fused(const infv2_problem& p, const void* Q, const KeySet& ks,
                               float* S_cmp, int32_t* idx, int32_t* n_sel, void* ws, int n_blk,
                               float scale, int budget, hipStream_t stream) {
  if (!scores_use_split(p)) {
    ScoresArgs a = prefill_args(p, Q, ks, S_cmp, n_blk, scale);
    a.idx = idx;
    a.n_sel = n_sel;
    a.marks = (int32_t*)((char*)ws + align256(scores_workspace(p, ks)));
    a.k = p.k;
    a.N_init = p.N_init;
    a.N_local = p.N_local;
    a.budget = budget;
    launch_prefill_scores<true>(p, a, stream);
    return hipGetLastError();
  }
  return launch_select_split(p, Q, ks, nullptr, S_cmp, idx, n_sel, ws, n_blk, scale, budget,
                             stream);
}

// The decode selection with the step's append fused into the logits sweep:
// kernels [c1_begin, c1_end) of every sequence are formed from K inside the
// sweep and written to Kc1 (bit for bit what launch_compress_k writes).
// Requires scores_use_split(p), select_fused_shape(p, n_C1), exact LSE.
// With lists set, the selection stops at the per-chunk candidate lists (in
// ws; *lists says where): idx and n_sel are not written.
hipError_t launch_select_append(const infv2_problem& p, const void* Q, const void* K, void* Kc1,
                                int c1_begin, int c1_end, int64_t kv_cap, const KeySet& ks,
                                int32_t* idx, int32_t* n_sel, void* ws, int n_blk, float scale,
                                int budget, hipStream_t stream, CandLists* lists) {
  SplitArgs app = {};
  app.K = (const uint16_t*)K;
  app.Kc1_out = (uint16_t*)Kc1;
  app.kv_cap = kv_cap;
  app.app_begin = c1_begin;
  app.app_end = c1_end;
  app.l_C1 = p.l_C1;
  app.s_C1 = p.s_C1;
  app.inv_l1 = 1.0 / (double)p.l_C1;
  return launch_select_split(p, Q, ks, nullptr, nullptr, idx, n_sel, ws, n_blk, scale, budget,
                             stream, &app, lists);
}

// S_sh: S^shared [batch][h_kv][n_q][n_C1] as well, or null.
hipError_t launch_block_scores(const infv2_problem& p, const void* Q, const KeySet& ks,
                               float* S_cmp, float* S_sh, void* ws, int n_blk, float scale,
                               hipStream_t stream) {
  if (scores_use_split(p)) {
    SplitArgs a = split_args(p, Q, ks, S_cmp, ws, n_blk, scale);
    a.S_sh = S_sh;
    launch_split_scores(p, a, stream);
    return hipGetLastError();
  }
  if (scores_fast_shape(p)) {
    ScoresArgs a = prefill_args(p, Q, ks, S_cmp, n_blk, scale);
    a.S_sh = S_sh;
    launch_prefill_scores<false>(p, a, stream);
    return hipGetLastError();
  }
  GenericScoresArgs a = {};
  a.Q = Q;
  a.Kc1 = ks.Kc1;
  a.Kc2 = ks.Kc2;
  a.S_cmp = S_cmp;
  a.S_sh = S_sh;
  a.dtype = p.dtype;
  a.n_q = p.n_q;
  a.q_pos0 = p.q_pos0;
  a.h_kv = p.h_kv;
  a.G = p.G;
  a.d = p.d;
  a.n_c1 = ks.n_c1;
  a.n_c2 = ks.n_c2;
  a.n_blk = n_blk;
  a.B = p.B;
  a.l_C1 = p.l_C1;
  a.s_C1 = p.s_C1;
  a.approx = p.lse_approx;
  a.c1_cap = ks.c1_cap;
  a.c2_cap = ks.c2_cap;
  a.scale = scale;
  dim3 grid(p.n_q, p.h_kv, p.batch);
  const size_t lds = scores_generic_lds(p, ks.n_c1);
  if (p.dtype == INFV2_F32)
    hipLaunchKernelGGL(scores_generic_kernel<float>, grid, dim3(256), lds, stream, a);
  else
    hipLaunchKernelGGL(scores_generic_kernel<uint16_t>, grid, dim3(256), lds, stream, a);
  return hipGetLastError();
}

}  // namespace infv2
