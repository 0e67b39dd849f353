// Block-sparse attention over the selected blocks, and dense causal attention.
//
// paperlayer.ai summary of arXiv 2509.24663v1, "A IMPLEMENTATION DETAIL": queries
// are processed in parallel, the inner loop visits only the key blocks of the
// visible set, with FlashAttention-style online softmax; the kernel returns O
// and the log-sum-exp.  The key tile (64) equals the block size B, so B is a
// multiple of it.  Token-level query granularity (OpenBMB blog
// "技术Blog-4 | 新一代InfLLM：可训练的稀疏注意力机制", 查询和键值词元的不同粒度): every
// query token has its own block list, shared by the 16 heads of its group.
//
// bf16 kernels (G = 16, d = 128, B = 64):
//  * one wavefront per (token, group); the 16 heads are the N = 16 columns of
//    v_mfma_f32_16x16x32_bf16.  Scores are formed transposed, S^T = K Q^T
//    (keys on the M axis), so that each lane ends up holding 8 consecutive
//    keys of one head -- exactly the B-operand layout of the P V product
//    O^T = V^T P^T.  No cross-lane data movement besides the row max.
//  * prefill first writes K and V once in MFMA-fragment order (kv_pack_kernel)
//    so that every fragment load of the gather is one coalesced 1 KB load;
//    decode stages each selected block through LDS.
//  * prefill runs one wave per SIMD with two blocks of loads in flight ahead
//    of the math, and rescales O only when a head's running maximum grows by
//    more than 2^8;
//  * decode splits the selected blocks over workgroups (one block each) and
//    merges the partial (max, sum, O) afterwards; for a varlen batch each
//    sequence's positions come from a device array of lengths, and with a
//    paged cache each selected block is read from its page (page = block).
// A generic fp64 kernel serves fp32 I/O and other shapes.
#include <algorithm>

#include "attn_layout.hpp"
#include "select_merge.hpp"

// tokens per wave of the sparse prefill attention below the key-range split
// (1: attn_prefill_kernel; 2 or 4: attn_prefill_seq_kernel)
#ifndef INFV2_ATTN_TPW
#define INFV2_ATTN_TPW 2
#endif

namespace infv2 {


// ---------------------------------------------------------------------------
// K, V [b][kv_cap][h_kv][d] -> packs [b][h_kv][n_blk][16 fragments][64 lanes][8]
// (bf16), zero beyond n_kv.  Fragment f of a block is the 1 KB that one MFMA
// operand load needs, in lane order, so the attention kernel reads every
// fragment with one fully coalesced 16-byte-per-lane load:
//   K pack, f = 4t + ks:  lane l holds K[tile_key(t, l&15)][32ks + 8(l>>4) .. +7]
//   V pack, f = 2mt + ks: lane l holds V[32ks + 8(l>>4) .. +7][16mt + (l&15)]
// (A gather of rows straight into the operand layout would put 16 different
// rows on consecutive lanes and cost one address request per lane.)
// grid: x = blocks, y = h_kv, z = batch.  256 threads.
// ---------------------------------------------------------------------------

__global__ void __launch_bounds__(256) kv_pack_kernel(const uint16_t* __restrict__ K,
                                                      const uint16_t* __restrict__ V,
                                                      uint16_t* __restrict__ Kp,
                                                      uint16_t* __restrict__ Vp, int n_kv,
                                                      int n_blk, int h_kv, int64_t kv_cap) {
  __shared__ __attribute__((aligned(16))) uint16_t kt[AT_B][AT_D + 8];
  __shared__ __attribute__((aligned(16))) uint16_t vt[AT_B][AT_D + 8];
  const int blk = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int u = tid + 256 * i;
    const int r = u >> 4, c8 = (u & 15) * 8;
    const int tok = blk * AT_B + r;
    u32x4 kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
    if (tok < n_kv) {
      const size_t off = (((size_t)b * kv_cap + tok) * h_kv + g) * AT_D + c8;
      kv = *(const u32x4*)(K + off);
      vv = *(const u32x4*)(V + off);
    }
    *(u32x4*)&kt[r][c8] = kv;
    *(u32x4*)&vt[r][c8] = vv;
  }
  __syncthreads();
  const size_t base = (((size_t)b * h_kv + g) * n_blk + blk) * PACK_ELEMS;
  // 16 fragments x 64 lanes = 1024 pieces of 16 B per pack, 4 per thread;
  // K in the key layout, V in the feature layout
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int u = tid + 256 * i;
    *(u32x4*)(Kp + base + (size_t)u * 8) = pack_piece_keys(&kt[0][0], AT_D + 8, u);
    *(u32x4*)(Vp + base + (size_t)u * 8) = pack_piece_features(&vt[0][0], AT_D + 8, u);
  }
}

struct AttnArgs {
  const uint16_t* Q;
  const uint16_t* K;
  const uint16_t* Kp;     // prefill: K and V in fragment order (kv_pack_kernel)
  const uint16_t* Vp;
  const uint16_t* V;      // decode: natural V
  const int32_t* idx;     // nullptr -> dense
  const int32_t* n_sel;
  uint16_t* O;
  float* lse;
  float* part_o;          // decode partials
  float2* part_ml;
  int batch, n_q, q_pos0, n_kv, n_blk, h_kv, budget;
  int64_t kv_cap;
  float c;                // scale * log2(e)
  // decode of a varlen batch (null: every sequence has n_kv keys, queries
  // from q_pos0): sequence b holds seq_lens[b] keys, its queries are the last
  // n_q.  Paged cache (null: K, V [b][kv_cap][h_kv][d]): K, V are pools of
  // n_pages pages [B][h_kv][d]; block j of sequence b is page
  // block_table[b * max_blocks + j].
  const int32_t* seq_lens;
  const int32_t* block_table;
  int max_blocks, n_pages;
};

// Scores and online softmax of one 64-key block for one token's 16 heads.
// kf[t][ks]: K fragments (rows tile_key(t, lane&15), features 32ks+8*(lane>>4)).
// Returns P^T as two bf16 B operands (k-step ks = keys 32ks + 8*(lane>>4) ..+7)
// and rescales o / l_run when the running maximum moves.  The reference m_run
// is only raised when some head's block maximum exceeds it by more than 2^8
// (log2 units): probabilities then stay below 256, and O is rescaled rarely.
// DIAG: the block holds the query position; keys after p are masked.
template <bool DIAG>
__device__ __forceinline__ void attn_softmax(f32x4 (&s)[4], f32x4 (&o)[8], float& m_run,
                                             float& l_run, int kv0, int p, float c, int lane,
                                             bf16x8 (&pf)[2]);

template <bool DIAG>
__device__ __forceinline__ void attn_scores(const bf16x8 (&qf)[4], const bf16x8 (&kf)[4][4],
                                            f32x4 (&o)[8], float& m_run, float& l_run, int kv0,
                                            int p, float c, int lane, bf16x8 (&pf)[2]) {
  f32x4 s[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    s[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) s[t] = mfma16(kf[t][ks], qf[ks], s[t]);
  }
  attn_softmax<DIAG>(s, o, m_run, l_run, kv0, p, c, lane, pf);
}

// Online softmax of one 64-key block given its raw scores s (S^T tiles); the
// scale enters through the maximum and one fma per score in the exponent.
template <bool DIAG>
__device__ __forceinline__ void attn_softmax(f32x4 (&s)[4], f32x4 (&o)[8], float& m_run,
                                             float& l_run, int kv0, int p, float c, int lane,
                                             bf16x8 (&pf)[2]) {
  const int grp = lane >> 4;
  float mx = kNegInf;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float x = s[t][i];
      if constexpr (DIAG) {
        const int key = kv0 + 32 * (t >> 1) + 8 * grp + 4 * (t & 1) + i;
        if (key > p) x = kNegInf;
      }
      s[t][i] = x;
      mx = fmaxf(mx, x);
    }
  mx *= c;   // the maximum of the scaled scores (c > 0; -inf stays -inf)
  if (__ballot(mx > m_run + 8.0f)) {
    // (mx > m_run implies mx is finite)
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = fast_exp2(m_run - m_new);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) o[mt][i] *= alpha;
  }
  // before the first visible key m_run is -inf and every score here is -inf
  const float mref = (m_run == kNegInf) ? 0.f : m_run;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = 2 * ks + (e >> 1);
      const int i0 = 2 * (e & 1);
      const float p0 = fast_exp2(__builtin_fmaf(s[t][i0], c, -mref));
      const float p1 = fast_exp2(__builtin_fmaf(s[t][i0 + 1], c, -mref));
      l_run += p0 + p1;                      // fp32 sum: exact-to-fp32 LSE
      w[e] = pack_bf16x2(p0, p1);
    }
    pf[ks] = as_bf16x8(u32x4{w[0], w[1], w[2], w[3]});
  }
}

// O^T += V^T P^T for one block; vf[mt][ks]: V^T fragments (feature
// 16mt+(lane&15), keys 32ks+8*(lane>>4) .. +7).
__device__ __forceinline__ void attn_pv(const bf16x8 (&vf)[8][2], const bf16x8 (&pf)[2],
                                        f32x4 (&o)[8]) {
#pragma unroll
  for (int mt = 0; mt < 8; ++mt)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) o[mt] = mfma16(vf[mt][ks], pf[ks], o[mt]);
}

__device__ __forceinline__ void load_qfrag(const AttnArgs& a, int b, int t, int g, int lane,
                                           bf16x8 (&qf)[4]) {
  const int hq = a.h_kv * AT_G;
  const uint16_t* q = a.Q + (((size_t)b * a.n_q + t) * hq + g * AT_G + (lane & 15)) * AT_D;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
    qf[ks] = as_bf16x8(__builtin_nontemporal_load((const u32x4*)(q + 32 * ks + 8 * (lane >> 4))));
}

// 1-D grid, 16 workgroups (4 tokens each) per 64-token query block.
// Workgroups are dispatched round-robin over the 8 XCDs; the mapping below
// puts all 16 workgroups of one query block on the same XCD, so blocks that
// several of its tokens select are read once into that XCD's L2 (every token
// walks its ascending block list at about the same pace).  Late query blocks
// (long rows) go first.
// One wave per SIMD (the registers of two blocks' fragments, 512 per lane
// with the accumulation registers): fewer tokens in flight per CU keep the
// blocks they gather in L2 longer -- measured 2.03 -> 1.76 ms at 32k, 14.1 ->
// 12.9 ms at 128k against two waves per SIMD with one block in flight.
// Loads run two list entries ahead: after the scores of entry i its K set is
// refilled with entry i+2, after its PV the V set.
// LONG: block lists of more than 64 entries (budget and n_blk > 64) are re-read 64 at a
// time; the common case never touches memory for the list inside the loop.
template <bool SPARSE, bool LONG>
__global__ void __launch_bounds__(256, 1) attn_prefill_kernel(AttnArgs a) {
  // (the wave index and the list length are made uniform: a loop whose bound
  // the compiler takes as per-lane gets exec-masked paths, and the wait counts
  // of its loads become conservative)
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n_qb = (a.n_q + AT_B - 1) / AT_B;
  const int n_bg = a.batch * a.h_kv;
  const int bid = blockIdx.x;
  const int xcd = bid & 7, r = bid >> 3;
  const int qbg = (r >> 4) * 8 + xcd;                  // query block, global order
  if (qbg >= n_qb * n_bg) return;
  const int qb = n_qb - 1 - qbg / n_bg;                // late tokens (long rows) first
  const int bg = qbg % n_bg;
  const int g = bg % a.h_kv, b = bg / a.h_kv;
  const int t = qb * AT_B + (r & 15) * 4 + wave;
  if (t >= a.n_q) return;
  const int p = a.q_pos0 + t;
  const int b_p = p / AT_B;
  bf16x8 qf[4];
  load_qfrag(a, b, t, g, lane, qf);
  f32x4 o[8];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) o[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegInf, l_run = 0.f;
  const size_t row = ((size_t)b * a.h_kv + g) * a.n_q + t;
  const int32_t* sel = SPARSE ? a.idx + row * a.budget : nullptr;
  // (the first 64 entries are read with the length, not after it)
  const int raw0 = (SPARSE && lane < a.budget) ? sel[lane] : -1;
  const int nblocks = __builtin_amdgcn_readfirstlane(SPARSE ? a.n_sel[row] : b_p + 1);
  const size_t pack0 = ((size_t)b * a.h_kv + g) * a.n_blk * PACK_ELEMS + lane * 8;
  const uint16_t* kbase = a.Kp + pack0;
  const uint16_t* vbase = a.Vp + pack0;
  const int grp = lane >> 4, r16 = lane & 15;
  // The block list is held one entry per lane, 64 entries at a time, so that
  // reading the next entry (a uniform lane read) never waits on memory.
  int list_base = 0;
  int my_entry = lane < nblocks ? raw0 : -1;
  // block of list entry bi, or -1 when the entry is not a causal block
  auto block_at = [&](int bi) -> int {
    int blk = bi;
    if constexpr (SPARSE) {
      if constexpr (LONG) {
        if (bi >= list_base + 64) {
          list_base = bi & ~63;
          my_entry = (list_base + lane < nblocks) ? sel[list_base + lane] : -1;
        }
      }
      blk = __builtin_amdgcn_readlane(my_entry, bi - list_base);
    }
    return (blk < 0 || blk > b_p) ? -1 : blk;
  };
  // one coalesced 1 KB load per fragment (keys past n_kv are zero in the pack)
  auto load_k = [&](int blk, bf16x8 (&kf)[4][4]) {
    const uint16_t* src = kbase + (uint32_t)blk * PACK_ELEMS;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) kf[tt][ks] = as_bf16x8(*(const u32x4*)(src + (4 * tt + ks) * 512));
  };
  auto load_v = [&](int blk, bf16x8 (&vf)[8][2]) {
    const uint16_t* src = vbase + (uint32_t)blk * PACK_ELEMS;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) vf[mt][ks] = as_bf16x8(*(const u32x4*)(src + (2 * mt + ks) * 512));
  };
  // Two register sets (A: even list entries, B: odd ones): the K and V of
  // entries i+1 and i+2 are in flight while entry i is computed.  Inside the
  // loop every step issues its loads unconditionally (past the end, the last
  // entry's block again), so the loads in flight are the same on every path;
  // the loop has no other exit than its end test (an exit between the two
  // steps gives the compiler a path that skips set B's loads, and its wait
  // counts for set A turn conservative).  The pipeline is skewed by one
  // entry: step i issues the score MFMAs of entry i, then the P*V MFMAs of
  // entry i-1, then the softmax of entry i, so that with one wave per SIMD
  // neither the softmax nor a P*V waits on the MFMAs just before it; O, m and
  // l see the same operations in the same order as unskewed (bitwise the
  // same output).  Entry i's K set is refilled with entry i+2 after its score
  // MFMAs, entry i-1's V set with entry i+1 after its P*V.  A non-causal entry
  // is processed as block 0 with every key masked: it adds nothing.
  bf16x8 kA[4][4], vA[8][2], kB[4][4], vB[8][2], pf[2];
  auto score_mfma = [&](bf16x8 (&kf)[4][4], f32x4 (&sc)[4]) {
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      sc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) sc[tt] = mfma16(kf[tt][ks], qf[ks], sc[tt]);
    }
  };
  auto softmax_of = [&](int blk, f32x4 (&sc)[4]) {
    const int kv0 = max(blk, 0) * AT_B;
    if (blk == b_p)
      attn_softmax<true>(sc, o, m_run, l_run, kv0, p, a.c, lane, pf);
    else if (blk < 0)
      attn_softmax<true>(sc, o, m_run, l_run, kv0, -1, a.c, lane, pf);
    else
      attn_softmax<false>(sc, o, m_run, l_run, kv0, p, a.c, lane, pf);
  };
  auto step = [&](int blk, bf16x8 (&kx)[4][4], bf16x8 (&vy)[8][2], int nk, int nv) {
    f32x4 sc[4];
    score_mfma(kx, sc);
    load_k(max(nk, 0), kx);
    __builtin_amdgcn_sched_barrier(0);
    attn_pv(vy, pf, o);
    load_v(max(nv, 0), vy);
    __builtin_amdgcn_sched_barrier(0);
    softmax_of(blk, sc);
  };
  const int b0 = block_at(0);
  int bcur = block_at(min(1, nblocks - 1));
  // issued in the loop's order (the scheduling barriers keep the scheduler
  // from reordering them: the wait counts at the loop head merge this order
  // with the loop's, and any other order makes every step wait for all loads
  // in flight, the prefetch included)
  load_k(max(b0, 0), kA);
  __builtin_amdgcn_sched_barrier(0);
  load_v(max(b0, 0), vA);
  __builtin_amdgcn_sched_barrier(0);
  load_k(max(bcur, 0), kB);
  __builtin_amdgcn_sched_barrier(0);
  load_v(max(bcur, 0), vB);
  __builtin_amdgcn_sched_barrier(0);
  if (nblocks > 0) {
    // entry 0: scores and softmax (its P*V goes with entry 1)
    f32x4 sc[4];
    score_mfma(kA, sc);
    load_k(max(block_at(min(2, nblocks - 1)), 0), kA);
    __builtin_amdgcn_sched_barrier(0);
    softmax_of(b0, sc);
    int bi = 1;
    for (; bi + 1 < nblocks; bi += 2) {
      const int bnx = block_at(bi + 1);
      const int b2 = block_at(min(bi + 2, nblocks - 1));
      step(bcur, kB, vA, b2, bnx);
      step(bnx, kA, vB, block_at(min(bi + 3, nblocks - 1)), b2);
      bcur = b2;
    }
    if (bi < nblocks) {
      step(bcur, kB, vA, bcur, bcur);     // an odd last entry (set B)
      attn_pv(vB, pf, o);
    } else {
      attn_pv(vA, pf, o);                 // the last entry is even (set A)
    }
  }
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  const float inv = 1.0f / l_run;
  const int hq = a.h_kv * AT_G;
  uint16_t* orow = a.O + (((size_t)b * a.n_q + t) * hq + g * AT_G + r16) * AT_D;
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) {
    const uint32_t w0 = pack_bf16x2(o[mt][0] * inv, o[mt][1] * inv);
    const uint32_t w1 = pack_bf16x2(o[mt][2] * inv, o[mt][3] * inv);
    __builtin_nontemporal_store(u32x2{w0, w1}, (u32x2*)(orow + 16 * mt + 4 * grp));
  }
  if (a.lse && grp == 0)
    __builtin_nontemporal_store((m_run + fast_log2(l_run)) * kLn2,
                                a.lse + ((size_t)b * hq + g * AT_G + r16) * a.n_q + t);
}

// The sparse prefill (lists of at most 64 entries) with TPW consecutive
// tokens per wave, taken one after the other: the wave walks the pairs
// (token, list entry) of its tokens as one sequence, so that the loads run
// two pairs ahead across the token boundaries and the next token starts with
// its first blocks already in flight (a workgroup that starts cold waits a
// list read and a block read before its first MFMA).  Every token is computed
// exactly as in attn_prefill_kernel (same blocks, same order, same
// arithmetic): O and LSE are bitwise the same.  Q of the wave's tokens is
// staged in LDS; one wave per SIMD as there.
template <int TPW>
__global__ void __launch_bounds__(256, 1) attn_prefill_seq_kernel(AttnArgs a) {
  __shared__ u32x4 qlds[4][TPW][4][64];
  // (uniform wave index and counts, as in attn_prefill_kernel)
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n_qb = (a.n_q + AT_B - 1) / AT_B;
  const int n_bg = a.batch * a.h_kv;
  constexpr int WPQ = 16 / TPW;                        // workgroups per query block
  const int bid = blockIdx.x;
  const int xcd = bid & 7, r = bid >> 3;
  const int qbg = (r / WPQ) * 8 + xcd;                 // query block, global order
  if (qbg >= n_qb * n_bg) return;
  const int qb = n_qb - 1 - qbg / n_bg;                // late tokens (long rows) first
  const int bg = qbg % n_bg;
  const int g = bg % a.h_kv, b = bg / a.h_kv;
  const int t0 = qb * AT_B + (r % WPQ) * (4 * TPW) + wave * TPW;
  if (t0 >= a.n_q) return;
  const int hq = a.h_kv * AT_G;
  const int grp = lane >> 4, r16 = lane & 15;
  // the wave's tokens: list entry `lane` of token j in E[j], pair counts,
  // the pair index where each token starts; Q to LDS
  // (every read of the set-up -- entries, lengths, Q -- is issued before
  // the first is used: one memory round trip, not one after another; a
  // token past n_q reads token n_q - 1 and is never used)
  int E[TPW], start[TPW + 1], nsr[TPW];
  u32x4 qr[TPW][4];
#pragma unroll
  for (int j = 0; j < TPW; ++j) {
    const int t = min(t0 + j, a.n_q - 1);
    const size_t row = ((size_t)b * a.h_kv + g) * a.n_q + t;
    E[j] = lane < a.budget ? a.idx[row * a.budget + lane] : -1;
    nsr[j] = a.n_sel[row];
    const uint16_t* q = a.Q + (((size_t)b * a.n_q + t) * hq + g * AT_G + r16) * AT_D;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      qr[j][ks] = __builtin_nontemporal_load((const u32x4*)(q + 32 * ks + 8 * grp));
  }
  __builtin_amdgcn_sched_barrier(0);
  start[0] = 0;
#pragma unroll
  for (int j = 0; j < TPW; ++j) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qlds[wave][j][ks][lane] = qr[j][ks];
    const int nb = t0 + j < a.n_q ? __builtin_amdgcn_readfirstlane(min(nsr[j], a.budget)) : 0;
    E[j] = lane < nb ? E[j] : -1;
    start[j + 1] = start[j] + nb;
  }
  const int ntok = min(TPW, a.n_q - t0);
  const int total = start[TPW];
  auto token_of = [&](int i) -> int {                  // (uniform)
    int j = 0;
#pragma unroll
    for (int k = 1; k < TPW; ++k) j += (i >= start[k]) ? 1 : 0;
    return j;
  };
  // block of pair i, or -1 when the entry is not a causal block of its token
  auto block_at = [&](int i) -> int {
    const int j = token_of(i);
    int ev = E[0];
#pragma unroll
    for (int k = 1; k < TPW; ++k) ev = (j == k) ? E[k] : ev;
    const int blk = __builtin_amdgcn_readlane(ev, i - start[j]);
    const int bpj = (a.q_pos0 + t0 + j) / AT_B;
    return (blk < 0 || blk > bpj) ? -1 : blk;
  };
  const size_t pack0 = ((size_t)b * a.h_kv + g) * a.n_blk * PACK_ELEMS + lane * 8;
  const uint16_t* kbase = a.Kp + pack0;
  const uint16_t* vbase = a.Vp + pack0;
  auto load_k = [&](int blk, bf16x8 (&kf)[4][4]) {
    const uint16_t* src = kbase + (uint32_t)blk * PACK_ELEMS;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) kf[tt][ks] = as_bf16x8(*(const u32x4*)(src + (4 * tt + ks) * 512));
  };
  auto load_v = [&](int blk, bf16x8 (&vf)[8][2]) {
    const uint16_t* src = vbase + (uint32_t)blk * PACK_ELEMS;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) vf[mt][ks] = as_bf16x8(*(const u32x4*)(src + (2 * mt + ks) * 512));
  };
  // the current token's state
  bf16x8 qf[4];
  f32x4 o[8];
  float m_run = kNegInf, l_run = 0.f;
  int cur = -1, p = 0, b_p = 0;
  auto load_q = [&](int j) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qf[ks] = as_bf16x8(qlds[wave][j][ks][lane]);
  };
  auto reset_token = [&](int j) {
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) o[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run = kNegInf;
    l_run = 0.f;
    cur = j;
    p = a.q_pos0 + t0 + j;
    b_p = p / AT_B;
  };
  auto finish_token = [&]() {
    float l = l_run;
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    const float inv = 1.0f / l;
    const int t = t0 + cur;
    uint16_t* orow = a.O + (((size_t)b * a.n_q + t) * hq + g * AT_G + r16) * AT_D;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      const uint32_t w0 = pack_bf16x2(o[mt][0] * inv, o[mt][1] * inv);
      const uint32_t w1 = pack_bf16x2(o[mt][2] * inv, o[mt][3] * inv);
      __builtin_nontemporal_store(u32x2{w0, w1}, (u32x2*)(orow + 16 * mt + 4 * grp));
    }
    if (a.lse && grp == 0)
      __builtin_nontemporal_store((m_run + fast_log2(l)) * kLn2,
                                  a.lse + ((size_t)b * hq + g * AT_G + r16) * a.n_q + t);
  };
  // tokens without pairs: O and LSE as the one-token kernel leaves them for
  // an empty list (written here, so that the loop only ever moves forward to
  // a token that has pairs)
#pragma unroll
  for (int j = 0; j < TPW; ++j)
    if (j < ntok && start[j + 1] == start[j]) {
      reset_token(j);
      finish_token();
    }
  cur = -1;
  bf16x8 kA[4][4], vA[8][2], kB[4][4], vB[8][2], pf[2];
  auto score_mfma = [&](bf16x8 (&kf)[4][4], f32x4 (&sc)[4]) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      sc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) sc[t] = mfma16(kf[t][ks], qf[ks], sc[t]);
    }
  };
  auto softmax_of = [&](int blk, f32x4 (&sc)[4]) {
    const int kv0 = max(blk, 0) * AT_B;
    if (blk == b_p)
      attn_softmax<true>(sc, o, m_run, l_run, kv0, p, a.c, lane, pf);
    else if (blk < 0)
      attn_softmax<true>(sc, o, m_run, l_run, kv0, -1, a.c, lane, pf);
    else
      attn_softmax<false>(sc, o, m_run, l_run, kv0, p, a.c, lane, pf);
  };
  // The pipeline is skewed by one pair, as in attn_range_kernel: step i
  // issues the score MFMAs of pair i, then the P*V MFMAs of pair i-1, then
  // the softmax of pair i, so that with one wave per SIMD neither the
  // softmax nor a P*V waits on the MFMAs just before it.  Each token's O, m
  // and l see the same operations in the same order as unskewed: the output
  // is bitwise the same.  Pair i's K and V are in set (i even ? A : B); its K
  // set is refilled with pair i+2 after its score MFMAs, and pair i-1's V set
  // with pair i+1 after its P*V.  At a token change the new token's Q comes
  // in before pair i's score MFMAs, and the old token is finished after the
  // P*V of its last pair.
  auto step = [&](int i, int blk, bf16x8 (&kx)[4][4], bf16x8 (&vy)[8][2], int nk, int nv) {
    const int j = token_of(i);
    const bool sw = j != cur;
    if (sw) load_q(j);
    f32x4 sc[4];
    score_mfma(kx, sc);
    load_k(max(nk, 0), kx);
    __builtin_amdgcn_sched_barrier(0);
    attn_pv(vy, pf, o);
    load_v(max(nv, 0), vy);
    __builtin_amdgcn_sched_barrier(0);
    if (sw) {
      finish_token();
      reset_token(j);
    }
    softmax_of(blk, sc);
  };
  if (total == 0) return;
  // first loads in the loop's order (see attn_prefill_kernel)
  const int b0 = block_at(0);
  int bcur = block_at(min(1, total - 1));
  load_k(max(b0, 0), kA);
  __builtin_amdgcn_sched_barrier(0);
  load_v(max(b0, 0), vA);
  __builtin_amdgcn_sched_barrier(0);
  load_k(max(bcur, 0), kB);
  __builtin_amdgcn_sched_barrier(0);
  load_v(max(bcur, 0), vB);
  __builtin_amdgcn_sched_barrier(0);
  {
    // pair 0: its token, scores and softmax (its P*V goes with pair 1)
    const int j = token_of(0);
    load_q(j);
    reset_token(j);
    f32x4 sc[4];
    score_mfma(kA, sc);
    load_k(max(block_at(min(2, total - 1)), 0), kA);
    __builtin_amdgcn_sched_barrier(0);
    softmax_of(b0, sc);
  }
  // whole pairs of steps (B: odd pairs, A: even ones); no exit in between
  int bi = 1;
  for (; bi + 1 < total; bi += 2) {
    const int bnx = block_at(bi + 1);
    const int b2 = block_at(min(bi + 2, total - 1));
    step(bi, bcur, kB, vA, b2, bnx);
    step(bi + 1, bnx, kA, vB, block_at(min(bi + 3, total - 1)), b2);
    bcur = b2;
  }
  if (bi < total) {
    // an odd last pair (set B), with nothing left to load
    step(bi, bcur, kB, vA, bcur, bcur);
    attn_pv(vB, pf, o);
  } else {
    attn_pv(vA, pf, o);                 // the last pair is even (set A)
  }
  finish_token();
}

// ---------------------------------------------------------------------------
// Key-range split of the sparse prefill attention.
//
// With per-token selections spread over the whole causal prefix, a
// token-major gather re-reads K/V blocks from wherever they happen to live:
// at 131072 keys the packs of one group (64 MB) are 16x one XCD's L2, and
// every L2 miss is served at ~7 TB/s whether or not the data sits in the
// Infinity Cache.  Here the keys are split into ranges of W blocks (W = 128:
// 4 MB of packs per group, one XCD's L2; 160 or 192 run ~3% faster but move
// 39% / 73% more bytes past L2) and a work item is (sequence, group,
// range r, tile of query tokens): it attends each token of the tile to its
// selected blocks inside range r only.  Work items are numbered range by
// range and every XCD takes a contiguous stretch of the numbering, so an XCD
// works through one range at a time and its gathers hit L2.
//
// A token whose blocks all lie in one range gets its output here; any other
// token leaves one partial per range it touches -- the running maximum m and
// sum l of every head (log2 domain, as in attn_softmax) and O/l rounded to
// bf16 -- in slot (rank of r among the token's ranges), and the merge
// combines them (in the tail rounds of the next query chunk's launch, the
// last chunk's in attn_range_merge_kernel):
//   M = max_s m_s,  L = sum_s l_s 2^(m_s - M),  O = sum_s (l_s 2^(m_s - M) / L) O_s.
// (The one extra bf16 rounding of each partial adds at most 2^-8 of that
// partial's magnitude, a convex combination of V rows, before the final
// rounding of O.)
//
// Per wave: TPW consecutive query tokens.  Their block lists (ascending) are
// read once; the entries inside range r form one contiguous run per token,
// found with ballots, and all (token, block) pairs of the wave are listed in
// LDS so that the loads run two pairs ahead across token boundaries, as in
// attn_prefill_kernel.  Q of the next token is loaded while the current one
// is computed.
// ---------------------------------------------------------------------------
constexpr int RG_WAVES = 4;
constexpr int RG_MAX_TPW = 4;             // tokens per wave (at most)
constexpr int RG_MAX_LIST = 64;           // block-list entries per token (budget)
constexpr int RG_PART_O_BYTES = AT_G * AT_D * 2;   // bf16 O of one (token, range)
constexpr int RG_PART_ML_BYTES = AT_G * 8;         // (m, l) per head

struct RangeArgs {
  AttnArgs a;
  u32x4* part_o;          // [rows][max_slots][4][64 lanes] x 16 B (bf16 O)
  float2* part_ml;        // [rows][max_slots][16]
  int W;                  // blocks per key range
  int tpw;                // tokens per wave
  int t_base, n_ct;       // first query token of this chunk, tokens in the chunk
  int n_qt;               // query tiles (RG_WAVES * tpw tokens) in the chunk
  int items_bg;           // work items per (sequence, group)
  int segment;            // work items per XCD
  int max_slots;          // partial slots per row
};

// First tile (within the chunk) whose last token reaches block r*W.
__device__ __host__ inline int rg_first_tile(int r, int W, int pos_base, int tile) {
  const int need = r * W * AT_B - pos_base - (tile - 1);
  return need <= 0 ? 0 : (need + tile - 1) / tile;
}

// Buffer descriptor over `bytes` bytes from `base` (raw, dword data): loads
// take their block offset in a scalar register and the lane's 16-byte offset
// in one vector register, and read 0 past `bytes`.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t pack_rsrc(const uint16_t* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, (int)bytes, 0x00020000);
}

// One work item of the range attention; bid plays the part of blockIdx.x
// (8 consecutive ids, one per XCD, form a round).  Run by workgroups of two
// per CU (two waves per SIMD, one block of K/V in registers per wave).
__device__ __forceinline__ void attn_range_item(const RangeArgs& ra, int bid) {
  const AttnArgs& a = ra.a;
  // Q fragments of the wave's tokens (the 4 k-steps of one token are 4 KB in
  // lane order) and the wave's (token << 16 | block) pairs
  __shared__ u32x4 qlds[RG_WAVES][RG_MAX_TPW][4][64];
  __shared__ int prs[RG_WAVES][RG_MAX_TPW * RG_MAX_LIST];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int item = (bid & 7) * ra.segment + (bid >> 3);
  if (item >= ra.items_bg * a.batch * a.h_kv) return;
  const int bg = item / ra.items_bg;
  int rem = item % ra.items_bg;
  const int tile = RG_WAVES * ra.tpw;
  const int pos_base = a.q_pos0 + ra.t_base;
  int r = 0, qt = 0;
  for (;; ++r) {
    const int first = rg_first_tile(r, ra.W, pos_base, tile);
    const int cnt = max(0, ra.n_qt - first);
    if (rem < cnt) {
      qt = first + rem;
      break;
    }
    rem -= cnt;
  }
  const int g = bg % a.h_kv, b = bg / a.h_kv;
  const int hq = a.h_kv * AT_G;
  const int tc0 = qt * tile + wave * ra.tpw;          // first chunk token of this wave
  // --- the wave's block lists: lane u holds entry u of token j in e[j]
  // (the list and its length are loaded together; entries past n_sel are
  // masked by the length below)
  int nsel_l = 0;
  if (lane < ra.tpw && tc0 + lane < ra.n_ct) {
    const size_t row = ((size_t)b * a.h_kv + g) * a.n_q + ra.t_base + tc0 + lane;
    nsel_l = min(a.n_sel[row], a.budget);
  }
  int e[RG_MAX_TPW];
#pragma unroll
  for (int j = 0; j < RG_MAX_TPW; ++j) {
    e[j] = -1;
    if (j < ra.tpw && tc0 + j < ra.n_ct && lane < a.budget) {
      const size_t row = ((size_t)b * a.h_kv + g) * a.n_q + ra.t_base + tc0 + j;
      e[j] = a.idx[row * a.budget + lane];
    }
  }
  // --- per token: the run inside range r, its slot, the token's range count
  int slot_l = 0, nparts_l = 0;                       // lane j holds token j's values
  int total = 0;
  uint32_t has_run = 0u;                              // bit j: token j has blocks in r
#pragma unroll
  for (int j = 0; j < RG_MAX_TPW; ++j) {
    if (j >= ra.tpw) break;
    const int nsj = __builtin_amdgcn_readlane(nsel_l, j);
    const int p = pos_base + tc0 + j;
    const int b_p = p / AT_B;
    const bool ok = lane < nsj && e[j] >= 0 && e[j] <= b_p;
    const int rg = ok ? e[j] / ra.W : 0x7fffffff;
    const int prev = __shfl_up(rg, 1, 64);
    const bool first = ok && (lane == 0 || rg != prev);
    const int s = __builtin_popcountll(__ballot(rg < r));
    const int c = __builtin_popcountll(__ballot(rg == r));
    const int sl = __builtin_popcountll(__ballot(first && rg < r));
    const int np = __builtin_popcountll(__ballot(first));
    if (lane == j) {
      slot_l = sl;
      nparts_l = np;
    }
    // pairs of token j: (j << 16) | block, blocks of the run in order (a
    // list that breaks the ascending-causal contract still reads blocks
    // within 0..b_p only)
    const int blk = __shfl(e[j], min(s + lane, 63), 64);
    if (lane < c) prs[wave][total + lane] = (j << 16) | min(max(blk, 0), b_p);
    total += c;
    has_run |= (c > 0 ? 1u : 0u) << j;
  }
  if (total == 0) return;                             // (no barrier below)
  // Q of the wave's tokens into registers now, to LDS once the first pair's
  // K and V loads are issued: the Q and K/V round trips overlap.  The loads
  // go through a buffer descriptor over the wave's tokens; a token without a
  // run in r gets an offset past its end, which reads 0 without a memory
  // access (one in six tokens at 128k), and every load is still issued, so
  // the waits stay exact.  A token past the chunk reads the chunk's last.
  u32x4 qr[RG_MAX_TPW][4];
  {
    // (wave-uniform: the descriptor lives in scalar registers)
    const int tq0 = __builtin_amdgcn_readfirstlane(ra.t_base + tc0);
    const int nt = __builtin_amdgcn_readfirstlane(min(ra.tpw, ra.n_ct - tc0));
    const uint32_t tok_bytes = (uint32_t)hq * AT_D * 2;
    const __amdgpu_buffer_rsrc_t rq = pack_rsrc(a.Q + ((size_t)b * a.n_q + tq0) * hq * AT_D,
                                                (uint32_t)nt * tok_bytes);
    const uint32_t lane_off_q = ((uint32_t)(g * AT_G + (lane & 15)) * AT_D + 8 * (lane >> 4)) * 2;
#pragma unroll
    for (int j = 0; j < RG_MAX_TPW; ++j) {
      if (j >= ra.tpw) break;
      const uint32_t off = ((has_run >> j) & 1u) ? (uint32_t)min(j, nt - 1) * tok_bytes + lane_off_q
                                                 : 0x80000000u;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        qr[j][ks] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rq, off, 64 * ks, 2));
    }
  }
  const size_t pack0 = ((size_t)b * a.h_kv + g) * a.n_blk * PACK_ELEMS;
  const uint32_t pack_bytes = (uint32_t)a.n_blk * PACK_ELEMS * 2;
  const __amdgpu_buffer_rsrc_t rk = pack_rsrc(a.Kp + pack0, pack_bytes);
  const __amdgpu_buffer_rsrc_t rv = pack_rsrc(a.Vp + pack0, pack_bytes);
  const int lane_off = lane * 16;
  const int grp = lane >> 4, r16 = lane & 15;
  // fragment f of block blk: 1 KB at blk * 16 KB + f * 1 KB, lane l's 16 B at l * 16
  auto load_k = [&](int blk, bf16x8 (&kf)[4][4]) {
    const int so = blk * (PACK_ELEMS * 2);
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        kf[tt][ks] = __builtin_bit_cast(
            bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rk, lane_off, so + (4 * tt + ks) * 1024, 0));
  };
  auto load_v = [&](int blk, bf16x8 (&vf)[8][2]) {
    const int so = blk * (PACK_ELEMS * 2);
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        vf[mt][ks] = __builtin_bit_cast(
            bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rv, lane_off, so + (2 * mt + ks) * 1024, 0));
  };
  // the pair list, 64 entries per lane register at a time (reading the next
  // pair is a lane read; the list is re-read from LDS every 64 pairs)
  int pbase = 0;
  int preg = prs[wave][min(lane, total - 1)];
  auto pair_at = [&](int i) -> int {
    i = min(i, total - 1);
    if (i >= pbase + 64) {
      pbase = i & ~63;
      preg = prs[wave][min(pbase + lane, total - 1)];
    }
    return __builtin_amdgcn_readlane(preg, i - pbase);
  };
  bf16x8 qc[4];
  auto load_q = [&](int j) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qc[ks] = as_bf16x8(qlds[wave][j][ks][lane]);
  };
  f32x4 o[8];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) o[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegInf, l_run = 0.f;
  int cur = pair_at(0);
  int tok = cur >> 16;
  int p_tok = pos_base + tc0 + tok;
  int bp_tok = p_tok / AT_B;
  // finish the current token: its output (one range) or its partial
  auto finish = [&]() {
    float l = l_run;
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    const float inv = 1.0f / l;
    const int tq = ra.t_base + tc0 + tok;
    const int np = __builtin_amdgcn_readlane(nparts_l, tok);
    if (np <= 1) {
      uint16_t* orow = a.O + (((size_t)b * a.n_q + tq) * hq + g * AT_G + r16) * AT_D;
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        const uint32_t w0 = pack_bf16x2(o[mt][0] * inv, o[mt][1] * inv);
        const uint32_t w1 = pack_bf16x2(o[mt][2] * inv, o[mt][3] * inv);
        __builtin_nontemporal_store(u32x2{w0, w1}, (u32x2*)(orow + 16 * mt + 4 * grp));
      }
      if (a.lse && grp == 0)
        __builtin_nontemporal_store((m_run + fast_log2(l)) * kLn2,
                                    a.lse + ((size_t)b * hq + g * AT_G + r16) * a.n_q + tq);
    } else {
      const int slot = __builtin_amdgcn_readlane(slot_l, tok);
      const size_t prow = (((size_t)b * a.h_kv + g) * ra.n_ct + tc0 + tok) * ra.max_slots + slot;
      // piece q of the lane: features 16 mt + 4 grp + i for mt = 2q, 2q + 1
      u32x4* dst = ra.part_o + prow * 256 + lane;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int m0 = 2 * q, m1 = 2 * q + 1;
        __builtin_nontemporal_store(
            u32x4{pack_bf16x2(o[m0][0] * inv, o[m0][1] * inv), pack_bf16x2(o[m0][2] * inv, o[m0][3] * inv),
                  pack_bf16x2(o[m1][0] * inv, o[m1][1] * inv), pack_bf16x2(o[m1][2] * inv, o[m1][3] * inv)},
            dst + 64 * q);
      }
      if (grp == 0)
        __builtin_nontemporal_store(f32x2{m_run, l}, (f32x2*)(ra.part_ml + prow * AT_G + r16));
    }
  };
  bf16x8 kf[4][4], vf[8][2], pf[2];
  load_k(cur & 0xffff, kf);                           // (in the loop's order)
  __builtin_amdgcn_sched_barrier(0);
  load_v(cur & 0xffff, vf);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < RG_MAX_TPW; ++j) {
    if (j >= ra.tpw) break;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qlds[wave][j][ks][lane] = qr[j][ks];
  }
  load_q(tok);
  // The pipeline is skewed by one pair: step i issues the score MFMAs of
  // pair i, then the P*V MFMAs of pair i-1, then the softmax of pair i, so
  // that neither the softmax (which reads the score MFMAs' results) nor a
  // P*V (which reads the softmax's probabilities) waits on the instruction
  // just before it.  Every token's O, m and l see the same operations in the
  // same order as unskewed (softmax i, P*V i, softmax i+1, ...): the output
  // is bitwise the same.  Each tile's K fragments are refilled with the next
  // pair's as soon as its MFMAs have issued, each V fragment with pair i's
  // after the P*V of pair i-1 has read it.  The refills are unconditional
  // (the last pair re-reads its own block): a load under a branch makes the
  // compiler's waits count it as absent.
  auto scores_refill = [&](int so_next, f32x4 (&sc)[4]) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      sc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) sc[t] = mfma16(kf[t][ks], qc[ks], sc[t]);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        kf[t][ks] = __builtin_bit_cast(
            bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rk, lane_off, so_next + (4 * t + ks) * 1024, 0));
    }
  };
  auto softmax_of = [&](int blk, f32x4 (&sc)[4]) {
    const int kv0 = blk * AT_B;
    if (blk == bp_tok)
      attn_softmax<true>(sc, o, m_run, l_run, kv0, p_tok, a.c, lane, pf);
    else
      attn_softmax<false>(sc, o, m_run, l_run, kv0, p_tok, a.c, lane, pf);
  };
  {
    // pair 0: scores and softmax (its P*V goes with the next step)
    const int nx = pair_at(1);
    f32x4 sc[4];
    scores_refill((nx & 0xffff) * (PACK_ELEMS * 2), sc);
    __builtin_amdgcn_sched_barrier(0);
    softmax_of(cur & 0xffff, sc);
    cur = nx;
  }
  for (int i = 1; i < total; ++i) {
    const int nx = pair_at(i + 1);
    const int blk = cur & 0xffff, tk = cur >> 16;
    if (tk != tok) load_q(tk);        // (O, m and l are still the previous token's)
    f32x4 sc[4];
    scores_refill((nx & 0xffff) * (PACK_ELEMS * 2), sc);
    __builtin_amdgcn_sched_barrier(0);
    const int so_cur = blk * (PACK_ELEMS * 2);
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) o[mt] = mfma16(vf[mt][ks], pf[ks], o[mt]);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        vf[mt][ks] = __builtin_bit_cast(
            bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rv, lane_off, so_cur + (2 * mt + ks) * 1024, 0));
    }
    __builtin_amdgcn_sched_barrier(0);
    if (tk != tok) {
      finish();
      tok = tk;
      p_tok = pos_base + tc0 + tok;
      bp_tok = p_tok / AT_B;
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) o[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      m_run = kNegInf;
      l_run = 0.f;
    }
    softmax_of(blk, sc);
    cur = nx;
  }
  // P*V of the last pair, then its token's output
#pragma unroll
  for (int mt = 0; mt < 8; ++mt)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) o[mt] = mfma16(vf[mt][ks], pf[ks], o[mt]);
  finish();
}

// Merge of the range partials of one (token, group) row: one wave per row,
// four rows per workgroup.  The row's range count comes from its block list
// (as in attn_range_kernel); rows with one range were written there.
__device__ __forceinline__ void attn_range_merge_rows(const RangeArgs& ra, int bid) {
  const AttnArgs& a = ra.a;
  const int lane = threadIdx.x & 63;
  const int rix = bid * 4 + (threadIdx.x >> 6);           // row in the chunk
  const int rows = a.batch * a.h_kv * ra.n_ct;
  if (rix >= rows) return;
  const int tc = rix % ra.n_ct, bg = rix / ra.n_ct;
  const int g = bg % a.h_kv, b = bg / a.h_kv;
  const int tq = ra.t_base + tc;
  const size_t row = ((size_t)b * a.h_kv + g) * a.n_q + tq;
  const int nsel = min(a.n_sel[row], a.budget);
  const int p = a.q_pos0 + tq;
  const int b_p = p / AT_B;
  const int ev = lane < nsel ? a.idx[row * a.budget + lane] : -1;
  const bool ok = lane < nsel && ev >= 0 && ev <= b_p;
  const int rg = ok ? ev / ra.W : 0x7fffffff;
  const int prev = __shfl_up(rg, 1, 64);
  const int np = __builtin_popcountll(__ballot(ok && (lane == 0 || rg != prev)));
  if (np <= 1) return;
  const int nparts = min(np, ra.max_slots);
  const size_t prow = ((size_t)bg * ra.n_ct + tc) * ra.max_slots;
  const int r16 = lane & 15, grp = lane >> 4;
  // one pass, four slots at a time, with the running maximum
  float M = kNegInf, L = 0.f;
  float acc[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) acc[i] = 0.f;
  for (int s0 = 0; s0 < nparts; s0 += 4) {
    u32x4 ov[4][4];
    float2 mlv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int s = min(s0 + u, nparts - 1);
      mlv[u] = ra.part_ml[(prow + s) * AT_G + r16];
      const u32x4* src = ra.part_o + (prow + s) * 256 + lane;
#pragma unroll
      for (int q = 0; q < 4; ++q) ov[u][q] = __builtin_nontemporal_load(src + 64 * q);
    }
    float mx = M;
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (s0 + u < nparts) mx = fmaxf(mx, mlv[u].x);
    const float wo = fast_exp2(M - mx);               // M = -inf gives 0
    L *= wo;
#pragma unroll
    for (int i = 0; i < 32; ++i) acc[i] *= wo;
    M = mx;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (s0 + u >= nparts) break;
      const float wgt = mlv[u].y * fast_exp2(mlv[u].x - M);
      L += wgt;
      // piece q word c: features 16 mt + 4 grp + {2(c&1), +1}, mt = 2q + (c >> 1)
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const uint32_t wd = ov[u][q][c];
          acc[8 * q + 2 * c] += wgt * bf16_bits_to_f32(wd & 0xffffu);
          acc[8 * q + 2 * c + 1] += wgt * bf16_bits_to_f32(wd >> 16);
        }
    }
  }
  const float inv = 1.0f / L;
  const int hq = a.h_kv * AT_G;
  uint16_t* orow = a.O + (((size_t)b * a.n_q + tq) * hq + g * AT_G + r16) * AT_D;
  // acc[4 mt + i] is feature 16 mt + 4 grp + i (the lane layout of o[mt][i])
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) {
    const uint32_t w0 = pack_bf16x2(acc[4 * mt] * inv, acc[4 * mt + 1] * inv);
    const uint32_t w1 = pack_bf16x2(acc[4 * mt + 2] * inv, acc[4 * mt + 3] * inv);
    __builtin_nontemporal_store(u32x2{w0, w1}, (u32x2*)(orow + 16 * mt + 4 * grp));
  }
  if (a.lse && grp == 0)
    a.lse[((size_t)b * hq + g * AT_G + r16) * a.n_q + tq] = (M + fast_log2(L)) * kLn2;
}

// The range attention of one query chunk, with the merge of the previous
// chunk's partials in the same launch, as its last rounds: the merge
// workgroups are dispatched once every range item has been, so they fill the
// range kernel's tail instead of running as a separate launch after it.
// (Spread evenly through the grid instead, they ran side by side with the
// range items the whole time and made the call slower: the partials they
// stream pass through the L2 that the gathers live on.)  The two chunks'
// partials sit in different buffers and their rows are disjoint.  The grid is
// rounds of 8 workgroups, one per XCD: the first total_rounds - merge_rounds
// keep the range kernel's item order per XCD, the rest merge 4 rows each.
__global__ void __launch_bounds__(256, 2) attn_range_kernel(RangeArgs ra, RangeArgs rm,
                                                            int merge_rounds, int total_rounds) {
  const int k = blockIdx.x >> 3, x = blockIdx.x & 7;
  const int range_rounds = total_rounds - merge_rounds;
  if (k < range_rounds)
    attn_range_item(ra, k * 8 + x);
  else
    attn_range_merge_rows(rm, (k - range_rounds) * 8 + x);
}

// The merge of the last chunk (nothing left to run beside it).
__global__ void __launch_bounds__(256) attn_range_merge_kernel(RangeArgs ra) {
  attn_range_merge_rows(ra, blockIdx.x);
}

// ---------------------------------------------------------------------------
// Dense causal attention (the dense switch): every token attends every causal
// block, so the blocks are shared.  A workgroup takes 16 consecutive query
// tokens of one group (8 waves x 2 tokens); each 64-key block is read once
// from the fragment-order packs into LDS (32 KB) and serves all 16 tokens;
// each wave reads a fragment from LDS once and applies it to both of its
// tokens.  Blocks from the first token's block on are masked per token (one
// block when the tile is aligned, two when q_pos0 is not a multiple of 16).
// Blocks are prefetched one ahead in registers.
// ---------------------------------------------------------------------------
constexpr int DN_TOK = 16;      // tokens per workgroup
constexpr int DN_WAVES = 8;     // 2 tokens per wave

__global__ void __launch_bounds__(512, 2) attn_dense_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t kvs[2][2 * PACK_ELEMS];   // 2 x 32 KB
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n_tiles = (a.n_q + DN_TOK - 1) / DN_TOK;
  const int n_bg = a.batch * a.h_kv;
  // XCD x takes (b, g) pairs with bg % 8 == x when possible; tiles of a pair
  // from the last (longest rows) to the first
  const int bid = blockIdx.x;
  const int xcd = bid & 7, r = bid >> 3;
  const int wi = r * 8 + xcd;                           // global work index
  if (wi >= n_tiles * n_bg) return;
  const int bg = wi % n_bg;
  const int tile = n_tiles - 1 - wi / n_bg;
  const int g = bg % a.h_kv, b = bg / a.h_kv;
  const int t0 = tile * DN_TOK;
  const int t_last = min(t0 + DN_TOK - 1, a.n_q - 1);
  const int b_last = (a.q_pos0 + t_last) / AT_B;        // the last token's block
  const int b_first = (a.q_pos0 + t0) / AT_B;           // the first token's block
  // this wave's tokens (past n_q: repeat the last token, never written)
  int tok[2], pos[2];
  bf16x8 qf[2][4];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    tok[u] = t0 + 2 * wave + u;
    pos[u] = a.q_pos0 + min(tok[u], a.n_q - 1);
    load_qfrag(a, b, min(tok[u], a.n_q - 1), g, lane, qf[u]);
  }
  f32x4 o[2][8];
  float m_run[2], l_run[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    m_run[u] = kNegInf;
    l_run[u] = 0.f;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) o[u][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // block staging: K pack then V pack, 2 x 16 KB, 4 pieces of 16 B per thread
  const size_t pack0 = ((size_t)b * a.h_kv + g) * a.n_blk * PACK_ELEMS;
  auto load_block = [&](int blk, u32x4 (&st)[4]) {
    const uint16_t* kp = a.Kp + pack0 + (size_t)blk * PACK_ELEMS;
    const uint16_t* vp = a.Vp + pack0 + (size_t)blk * PACK_ELEMS;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      st[i] = *(const u32x4*)(kp + (size_t)(tid + 512 * i) * 8);
      st[2 + i] = *(const u32x4*)(vp + (size_t)(tid + 512 * i) * 8);
    }
  };
  auto store_block = [&](int slot, const u32x4 (&st)[4]) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      *(u32x4*)&kvs[slot][(tid + 512 * i) * 8] = st[i];
      *(u32x4*)&kvs[slot][PACK_ELEMS + (tid + 512 * i) * 8] = st[2 + i];
    }
  };
  u32x4 st[4];
  load_block(0, st);
  store_block(0, st);
  if (b_last >= 1) load_block(1, st);
  __syncthreads();
  for (int blk = 0; blk <= b_last; ++blk) {
    const uint16_t* ks_ = &kvs[blk & 1][0];
    const uint16_t* vs_ = &kvs[blk & 1][PACK_ELEMS];
    const int kv0 = blk * AT_B;
    // scores S^T = K Q^T for both tokens, one K fragment read per (tile, k-step)
    f32x4 s[2][4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      bf16x8 kf[4];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) kf[ks] = as_bf16x8(*(const u32x4*)(ks_ + (4 * t + ks) * 512 + lane * 8));
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        s[u][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) s[u][t] = mfma16(kf[ks], qf[u][ks], s[u][t]);
      }
    }
    bf16x8 pf[2][2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if (blk >= b_first)   // blocks that hold a query position of the tile
        attn_softmax<true>(s[u], o[u], m_run[u], l_run[u], kv0, pos[u], a.c, lane, pf[u]);
      else
        attn_softmax<false>(s[u], o[u], m_run[u], l_run[u], kv0, pos[u], a.c, lane, pf[u]);
    }
    // O^T += V^T P^T for both tokens, one V fragment read per (d-tile, k-step)
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      bf16x8 vf[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) vf[ks] = as_bf16x8(*(const u32x4*)(vs_ + (2 * mt + ks) * 512 + lane * 8));
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) o[u][mt] = mfma16(vf[ks], pf[u][ks], o[u][mt]);
    }
    // next block into the other slot (its readers finished at the last barrier)
    if (blk + 1 <= b_last) {
      store_block((blk + 1) & 1, st);
      if (blk + 2 <= b_last) load_block(blk + 2, st);
    }
    __syncthreads();
  }
  const int grp = lane >> 4, r16 = lane & 15;
  const int hq = a.h_kv * AT_G;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    if (tok[u] >= a.n_q) continue;
    float l = l_run[u];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    const float inv = 1.0f / l;
    uint16_t* orow = a.O + (((size_t)b * a.n_q + tok[u]) * hq + g * AT_G + r16) * AT_D;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      const uint32_t w0 = pack_bf16x2(o[u][mt][0] * inv, o[u][mt][1] * inv);
      const uint32_t w1 = pack_bf16x2(o[u][mt][2] * inv, o[u][mt][3] * inv);
      __builtin_nontemporal_store(u32x2{w0, w1}, (u32x2*)(orow + 16 * mt + 4 * grp));
    }
    if (a.lse && grp == 0)
      __builtin_nontemporal_store((m_run[u] + fast_log2(l)) * kLn2,
                                  a.lse + ((size_t)b * hq + g * AT_G + r16) * a.n_q + tok[u]);
  }
}

// ---------------------------------------------------------------------------
// Decode: one workgroup (one wave) per (token, group, selected block).
// ---------------------------------------------------------------------------
// 8x8 transpose of bf16: in[r] holds 8 features of key r; out[q] gets feature
// q of keys 0..7.  v_perm_b32 picks 16-bit halves from two source dwords.
__device__ __forceinline__ void transpose8x8_bf16(const u32x4 (&in)[8], u32x4 (&out)[8]) {
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const uint32_t sel = (q & 1) ? 0x07060302u : 0x05040100u;
    uint32_t w[4];
#pragma unroll
    for (int m = 0; m < 4; ++m)
      w[m] = __builtin_amdgcn_perm(in[2 * m + 1][q >> 1], in[2 * m][q >> 1], sel);
    out[q] = u32x4{w[0], w[1], w[2], w[3]};
  }
}

// One 64-key block staged in LDS for the decode kernel.  Every global load is
// coalesced (lanes 16r..16r+15 read one 256-byte row).
//  K: natural rows, 16-byte chunk c of row r stored at chunk c ^ (r & 15).
//  V^T: vt2[key group kg][d'][8 keys] with d' = d ^ ((d >> 3) & 7); the 8x8
//  register transposes write it, and the fragment reads (8 keys of one
//  feature) read it, without bank conflicts.
__device__ __forceinline__ int vt_row(int d) { return d ^ ((d >> 3) & 7); }

// The split attention of one (token, group, list entry) once its block blk
// is known: the block's K and V through LDS, the scores, the softmax and P*V
// of its 64 keys, and the partial (O, max, sum) of every head at prow.
__device__ __forceinline__ void attn_split_block(const AttnArgs& a, int g, int b, size_t prow,
                                                 int blk, int n_kv, int p, const bf16x8 (&qf)[4],
                                                 uint8_t* kst, uint16_t (*vt2)[AT_D][8]) {
  const int lane = threadIdx.x;
  if (blk < 0 || blk > p / AT_B) {                  // only causal blocks
    if (lane < AT_G) a.part_ml[prow * AT_G + lane] = make_float2(kNegInf, 0.f);
    return;
  }
  const int kv0 = blk * AT_B;
  const size_t kstride = (size_t)a.h_kv * AT_D;
  // the block's first key row (a page of the pool, or rows of the sequence);
  // a page index out of the pool is clamped into it
  size_t row0 = (size_t)b * a.kv_cap + kv0;
  if (a.block_table)
    row0 = (size_t)min(max(a.block_table[(size_t)b * a.max_blocks + blk], 0), a.n_pages - 1) * AT_B;
  const uint16_t* kbase = a.K + row0 * kstride + (size_t)g * AT_D;
  const uint16_t* vbase = a.V + row0 * kstride + (size_t)g * AT_D;
  const int c = lane & 15, rq = lane >> 4;
  // rows past the last key are clamped to it (still in this block, as
  // kv0 <= p < n_kv); they lie after p: masked, P = 0
  const int r_last = n_kv - 1 - kv0;
  u32x4 kv[16], vin[2][8];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = min(4 * i + rq, r_last);
    kv[i] = *(const u32x4*)(kbase + (size_t)r * kstride + 8 * c);
  }
#pragma unroll
  for (int hh = 0; hh < 2; ++hh)
#pragma unroll
    for (int r8 = 0; r8 < 8; ++r8) {
      const int r = min(8 * (rq + 4 * hh) + r8, r_last);
      vin[hh][r8] = *(const u32x4*)(vbase + (size_t)r * kstride + 8 * c);
    }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int r = 4 * i + rq;
    *(u32x4*)(kst + r * (AT_D * 2) + ((c ^ (r & 15)) << 4)) = kv[i];
  }
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    u32x4 out[8];
    transpose8x8_bf16(vin[hh], out);
    const int kg = rq + 4 * hh;
#pragma unroll
    for (int q = 0; q < 8; ++q) *(u32x4*)&vt2[kg][vt_row(8 * c + q)][0] = out[q];
  }
  __syncthreads();
  f32x4 o[8];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) o[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegInf, l_run = 0.f;
  const int grp = lane >> 4, r16 = lane & 15;
  bf16x8 kf[4][4], vf[8][2];
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) {
    const int r = tile_key(tt, r16);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      kf[tt][ks] = as_bf16x8(*(const u32x4*)(kst + r * (AT_D * 2) + (((4 * ks + grp) ^ (r & 15)) << 4)));
  }
#pragma unroll
  for (int mt = 0; mt < 8; ++mt)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      vf[mt][ks] = as_bf16x8(*(const u32x4*)&vt2[4 * ks + grp][vt_row(16 * mt + r16)][0]);
  bf16x8 pf[2];
  if (blk == p / AT_B)
    attn_scores<true>(qf, kf, o, m_run, l_run, kv0, p, a.c, lane, pf);
  else
    attn_scores<false>(qf, kf, o, m_run, l_run, kv0, p, a.c, lane, pf);
  attn_pv(vf, pf, o);
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  // partial O^T (unnormalised) and (max, sum) per head
  float* po = a.part_o + prow * AT_G * AT_D;
#pragma unroll
  for (int mt = 0; mt < 8; ++mt)
    *(f32x4*)(po + (size_t)r16 * AT_D + 16 * mt + 4 * grp) = o[mt];
  if (grp == 0) a.part_ml[prow * AT_G + r16] = make_float2(m_run, l_run);
}

__global__ void __launch_bounds__(64) attn_split_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t kst[AT_B * AT_D * 2];
  __shared__ __attribute__((aligned(16))) uint16_t vt2[8][AT_D][8];
  const int lane = threadIdx.x;
  const int slot = blockIdx.x, g = blockIdx.y, bt = blockIdx.z;
  const int b = bt / a.n_q, t = bt % a.n_q;
  const size_t row = ((size_t)b * a.h_kv + g) * a.n_q + t;
  // the list length, the entry (slot < budget: in bounds), the sequence
  // length and Q are independent reads: all issued before the first use, so
  // that they cost one memory round trip, not one each
  const int nsel = a.n_sel[row];
  const int blk = a.idx[row * a.budget + slot];
  const int n_kv = a.seq_lens ? seq_len_of(a.seq_lens, b, a.n_q, a.n_kv) : a.n_kv;
  bf16x8 qf[4];
  load_qfrag(a, b, t, g, lane, qf);
  if (slot >= nsel) return;
  const int p = (a.seq_lens ? n_kv - a.n_q : a.q_pos0) + t;
  attn_split_block(a, g, b, row * a.budget + slot, blk, n_kv, p, qf, kst, vt2);
}

// The decode step's last selection stage and the split attention in one
// launch: every workgroup of a (token, group) row merges the row's per-chunk
// candidate lists itself (one wave, sel_merge_wave: the same set as
// scores_select_merge_kernel, ascending), takes the block of its own list
// entry and attends it; the row's entry-0 workgroup also writes idx and
// n_sel.  The separate merge launch and the round trip of idx between the
// two are gone.  One sequence length (no varlen, no paged cache).
struct DecodeSel {
  const uint64_t* cand;   // [rows][nch][kc] candidate keys (scores_split_pool_kernel)
  int32_t* idx;           // [rows][budget] out
  int32_t* n_sel;         // [rows] out
  int nch, kc, k, N_init, N_local;
};
__global__ void __launch_bounds__(64) attn_split_select_kernel(AttnArgs a, DecodeSel ds) {
  __shared__ __attribute__((aligned(16))) uint8_t kst[AT_B * AT_D * 2];
  __shared__ __attribute__((aligned(16))) uint16_t vt2[8][AT_D][8];
  __shared__ uint64_t pick[64];
  const int lane = threadIdx.x;
  const int slot = blockIdx.x, g = blockIdx.y, bt = blockIdx.z;
  const int b = bt / a.n_q, t = bt % a.n_q;
  const size_t row = ((size_t)b * a.h_kv + g) * a.n_q + t;
  bf16x8 qf[4];
  load_qfrag(a, b, t, g, lane, qf);
  const int p = a.q_pos0 + t;
  const RowSel rs = sel_merge_wave(ds.cand + row * (size_t)(ds.nch * ds.kc), ds.nch, ds.kc,
                                   ds.k, ds.N_init, ds.N_local, p / AT_B, lane, pick);
  if (slot == 0) {
    sel_write_list(rs, ds.idx + row * a.budget, a.budget, lane);
    if (lane == 0) ds.n_sel[row] = rs.n_sel;
  }
  if (slot >= rs.n_sel) return;
  attn_split_block(a, g, b, row * a.budget + slot, row_sel_block(rs, slot), a.n_kv, p, qf, kst,
                   vt2);
}

// grid: x = head within the group, y = h_kv, z = batch*n_q; 64 threads, two
// features each.  Slots are folded eight at a time, their loads in flight
// together; the weights rescale online when the running maximum moves.
constexpr int MERGE_SLOTS = 8;
__global__ void __launch_bounds__(64) attn_merge_kernel(AttnArgs a) {
  const int h = blockIdx.x, g = blockIdx.y, bt = blockIdx.z;
  const int b = bt / a.n_q, t = bt % a.n_q;
  const size_t row = ((size_t)b * a.h_kv + g) * a.n_q + t;
  const int nsel = a.n_sel[row];
  const int d0 = threadIdx.x * 2;
  float m = kNegInf, l = 0.f, acc0 = 0.f, acc1 = 0.f;
  for (int s0 = 0; s0 < nsel; s0 += MERGE_SLOTS) {
    float2 ml[MERGE_SLOTS], ov[MERGE_SLOTS];
#pragma unroll
    for (int u = 0; u < MERGE_SLOTS; ++u) {
      const size_t slot = row * a.budget + min(s0 + u, nsel - 1);
      ml[u] = a.part_ml[slot * AT_G + h];
      ov[u] = *(const float2*)(a.part_o + (slot * AT_G + h) * AT_D + d0);
    }
    float mx = m;
#pragma unroll
    for (int u = 0; u < MERGE_SLOTS; ++u)
      if (s0 + u < nsel) mx = fmaxf(mx, ml[u].x);
    if (mx == kNegInf) continue;                 // nothing visible yet
    const float wo = fast_exp2(m - mx);          // m == -inf gives 0
    l *= wo;
    acc0 *= wo;
    acc1 *= wo;
#pragma unroll
    for (int u = 0; u < MERGE_SLOTS; ++u) {
      if (s0 + u >= nsel || ml[u].x == kNegInf) continue;
      const float wn = fast_exp2(ml[u].x - mx);
      l += ml[u].y * wn;
      acc0 += ov[u].x * wn;
      acc1 += ov[u].y * wn;
    }
    m = mx;
  }
  const float inv = 1.0f / l;
  const int hq = a.h_kv * AT_G;
  uint16_t* orow = a.O + (((size_t)b * a.n_q + t) * hq + g * AT_G + h) * AT_D + d0;
  *(uint32_t*)orow = pack_bf16x2(acc0 * inv, acc1 * inv);
  if (a.lse && threadIdx.x == 0)
    a.lse[((size_t)b * hq + g * AT_G + h) * a.n_q + t] = (m + fast_log2(l)) * kLn2;
}

// ---------------------------------------------------------------------------
// Generic attention: any G, d <= 256, any B, fp32 or bf16 I/O; fp64 math.
// One workgroup per (token, group); keys processed 256 at a time.
// ---------------------------------------------------------------------------
struct GenericAttnArgs {
  const void* Q;
  const void* K;
  const void* V;
  const int32_t* idx;
  const int32_t* n_sel;
  void* O;
  float* lse;
  int dtype, n_q, q_pos0, n_kv, h_kv, G, d, B, budget;
  int64_t kv_cap;
  double scale;
};

template <typename T> __device__ __forceinline__ double ldv(const T* p, size_t i);
template <> __device__ __forceinline__ double ldv<float>(const float* p, size_t i) { return p[i]; }
template <> __device__ __forceinline__ double ldv<uint16_t>(const uint16_t* p, size_t i) {
  return (double)bf16_bits_to_f32(p[i]);
}

__device__ double bmax(double v, double* red) {
  for (int o = 32; o > 0; o >>= 1) v = fmax(v, __shfl_xor(v, o, 64));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  double r = red[0];
  for (int i = 1; i < (int)(blockDim.x >> 6); ++i) r = fmax(r, red[i]);
  return r;
}
__device__ double bsum(double v, double* red) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  double r = 0.0;
  for (int i = 0; i < (int)(blockDim.x >> 6); ++i) r += red[i];
  return r;
}

// fp64 -> bf16 bits, one rounding to nearest even (finite, normal-range data)
__device__ __forceinline__ uint16_t f64_to_bf16_bits(double x) {
  uint64_t u = __double_as_longlong(x);
  const uint64_t lsb = (u >> 45) & 1ull;
  u += 0x0000100000000000ull - 1ull + lsb;      // 2^44 - 1 + lsb
  u &= ~((1ull << 45) - 1ull);
  return (uint16_t)(__float_as_uint((float)__longlong_as_double(u)) >> 16);
}

template <typename T, bool SPARSE>
__global__ void __launch_bounds__(256) attn_generic_kernel(GenericAttnArgs a) {
  __shared__ double pz[256];
  __shared__ double red[8];
  const int t = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int p = a.q_pos0 + t;
  const int b_p = p / a.B;
  const size_t row = ((size_t)b * a.h_kv + g) * a.n_q + t;
  const int nblocks = SPARSE ? a.n_sel[row] : b_p + 1;
  const int32_t* sel = SPARSE ? a.idx + row * a.budget : nullptr;
  const int nkeys = nblocks * a.B;
  const T* Q = (const T*)a.Q;
  const T* K = (const T*)a.K;
  const T* V = (const T*)a.V;
  const int hq = a.h_kv * a.G;
  const size_t kstride = (size_t)a.h_kv * a.d;
  for (int h = 0; h < a.G; ++h) {
    const int head = g * a.G + h;
    const T* q = Q + (((size_t)b * a.n_q + t) * hq + head) * a.d;
    double m = -__builtin_huge_val(), l = 0.0, acc = 0.0;   // acc: feature threadIdx.x
    for (int base = 0; base < nkeys; base += 256) {
      const int i = base + threadIdx.x;
      double z = -__builtin_huge_val();
      if (i < nkeys) {
        const int blk = SPARSE ? sel[i / a.B] : i / a.B;
        const int tok = blk * a.B + i % a.B;
        if (blk >= 0 && tok <= p) {
          const T* kr = K + ((size_t)b * a.kv_cap + tok) * kstride + (size_t)g * a.d;
          double dot = 0.0;
          for (int e = 0; e < a.d; ++e) dot += ldv<T>(q, e) * ldv<T>(kr, e);
          z = dot * a.scale;
        }
      }
      const double cm = bmax(z, red);
      const double m_new = fmax(m, cm);
      const double alpha = (m == -__builtin_huge_val()) ? 0.0 : exp(m - m_new);
      const double pv = (z == -__builtin_huge_val()) ? 0.0 : exp(z - m_new);
      pz[threadIdx.x] = pv;
      const double cs = bsum(pv, red);          // includes a barrier after pz writes
      l = l * alpha + cs;
      acc *= alpha;
      if ((int)threadIdx.x < a.d) {
        const int lim = min(256, nkeys - base);
        for (int kk = 0; kk < lim; ++kk) {
          const double w = pz[kk];
          if (w == 0.0) continue;
          const int ii = base + kk;
          const int blk = SPARSE ? sel[ii / a.B] : ii / a.B;
          const int tok = blk * a.B + ii % a.B;
          acc += w * ldv<T>(V + ((size_t)b * a.kv_cap + tok) * kstride + (size_t)g * a.d,
                            threadIdx.x);
        }
      }
      m = m_new;
      __syncthreads();
    }
    if ((int)threadIdx.x < a.d) {
      const double o = acc / l;
      const size_t oi = (((size_t)b * a.n_q + t) * hq + head) * a.d + threadIdx.x;
      if (a.dtype == INFV2_F32) ((float*)a.O)[oi] = (float)o;
      else ((uint16_t*)a.O)[oi] = f64_to_bf16_bits(o);
    }
    if (a.lse && threadIdx.x == 0) a.lse[((size_t)b * hq + head) * a.n_q + t] = (float)(m + log(l));
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
bool attn_fast_shape(const infv2_problem& p) {
  return p.dtype == INFV2_BF16 && p.G == AT_G && p.d == AT_D && p.B == AT_B;
}
bool attn_use_split(const infv2_problem& p) { return attn_fast_shape(p) && p.n_q <= 4; }

// The key-range split of the sparse prefill attention (attn_range_kernel):
// range width, partial slots per row and the query chunk whose partials fit
// the workspace bound.  Used when the lists fit the kernel's LDS and blocks
// fit 16 bits.
#ifndef INFV2_RG_W_BLOCKS
#define INFV2_RG_W_BLOCKS 128
#endif
#ifndef INFV2_RG_SPLIT_MIN_BLOCKS
#define INFV2_RG_SPLIT_MIN_BLOCKS 1024
#endif
constexpr int RG_W_BLOCKS = INFV2_RG_W_BLOCKS;          // 4 MB of K+V packs per group
// the keys are split only from this many blocks on (below, one range)
constexpr int RG_SPLIT_MIN_BLOCKS = INFV2_RG_SPLIT_MIN_BLOCKS;
#ifndef INFV2_RG_PART_MIB
#define INFV2_RG_PART_MIB 1024
#endif
constexpr size_t RG_PART_BUDGET = (size_t)INFV2_RG_PART_MIB << 20;   // bytes of one chunk's partials (at most)
struct RangePlan {
  bool use;
  int W, R, max_slots, tpw, chunk;
};
static RangePlan range_plan(const infv2_problem& p, int budget) {
  RangePlan pl{};
  const int n_blk = (p.n_kv + AT_B - 1) / AT_B;
  // below RG_SPLIT_MIN_BLOCKS the token-major kernel (attn_prefill_kernel) is
  // faster: the packs mostly stay in L2 and a range split would only add the
  // per-(token, range) set-up and the merge
  pl.use = budget <= RG_MAX_LIST && n_blk < 65536 && n_blk >= RG_SPLIT_MIN_BLOCKS;
  if (!pl.use) return pl;
  pl.W = RG_W_BLOCKS;
  pl.R = (n_blk + pl.W - 1) / pl.W;
  pl.max_slots = pl.R > 1 ? std::min(pl.R, budget) : 0;
  // RG_MAX_TPW tokens per wave; fewer when that would leave the chip with
  // too few workgroups
  const long tiles16 = (long)p.batch * p.h_kv * ((p.n_q + 63) / 64);
  pl.tpw = tiles16 >= 1024 ? RG_MAX_TPW : 4;
  const int tile = RG_WAVES * pl.tpw;
  pl.chunk = p.n_q;
  if (pl.R > 1) {
    const size_t per_tok = (size_t)p.batch * p.h_kv * pl.max_slots *
                           (RG_PART_O_BYTES + RG_PART_ML_BYTES);
    const size_t fit = RG_PART_BUDGET / per_tok;
    if (fit < (size_t)p.n_q) pl.chunk = std::max(tile, (int)(fit / tile) * tile);
  }
  return pl;
}
// Bytes of one chunk's partial buffer (O pieces, then (m, l)).
static size_t range_buf_bytes(const infv2_problem& p, const RangePlan& pl) {
  const size_t slots = (size_t)p.batch * p.h_kv * pl.chunk * pl.max_slots;
  return ((slots * RG_PART_O_BYTES + 255) / 256 * 256 + slots * RG_PART_ML_BYTES + 255) / 256 * 256;
}
// Two buffers when the queries take several chunks: chunk i writes buffer
// i & 1 while the merge of chunk i - 1 reads the other.
static size_t range_part_bytes(const infv2_problem& p, const RangePlan& pl) {
  if (!pl.use || pl.R <= 1) return 0;
  return range_buf_bytes(p, pl) * (pl.chunk < p.n_q ? 2 : 1);
}

size_t attn_workspace(const infv2_problem& p, int budget, bool sparse) {
  if (!attn_fast_shape(p)) return 0;
  if (sparse && attn_use_split(p)) {
    const size_t slots = (size_t)p.batch * p.h_kv * p.n_q * budget;
    return slots * AT_G * AT_D * sizeof(float) + slots * AT_G * sizeof(float2);
  }
  const size_t n_blk = ((size_t)p.n_kv + AT_B - 1) / AT_B;
  const size_t packs = 2 * (size_t)p.batch * p.h_kv * n_blk * PACK_ELEMS * sizeof(uint16_t);
  if (!sparse) return packs;
  return packs + range_part_bytes(p, range_plan(p, budget));
}

// The range-split attention over one query chunk at a time (the partial
// slots are reused by the next chunk after its merge).
static void launch_attn_ranges(const infv2_problem& p, const AttnArgs& a, void* part_ws,
                               const RangePlan& pl, hipStream_t stream) {
  RangeArgs ra;
  ra.a = a;
  ra.W = pl.W;
  ra.tpw = pl.tpw;
  ra.max_slots = std::max(pl.max_slots, 1);
  const size_t slots = (size_t)p.batch * p.h_kv * pl.chunk * pl.max_slots;
  const size_t buf = range_buf_bytes(p, pl);
  auto use_buffer = [&](RangeArgs& r, int i) {
    char* base = (char*)part_ws + (i & 1) * buf;
    r.part_o = (u32x4*)base;
    r.part_ml = (float2*)(base + (slots * RG_PART_O_BYTES + 255) / 256 * 256);
  };
  const int tile = RG_WAVES * pl.tpw;
  RangeArgs rm = ra;               // the previous chunk, whose partials are merged
  int merge_rows = 0;              // 0: nothing to merge
  int i = 0;
  for (int t0 = 0; t0 < p.n_q; t0 += pl.chunk, ++i) {
    ra.t_base = t0;
    ra.n_ct = std::min(pl.chunk, p.n_q - t0);
    ra.n_qt = (ra.n_ct + tile - 1) / tile;
    use_buffer(ra, i);
    const int pos_base = p.q_pos0 + t0;
    const int last_rg = ((pos_base + ra.n_ct - 1) / AT_B) / pl.W;
    long items = 0;
    for (int r = 0; r <= last_rg; ++r)
      items += std::max(0, ra.n_qt - rg_first_tile(r, pl.W, pos_base, tile));
    ra.items_bg = (int)items;
    const long total = items * p.batch * p.h_kv;
    ra.segment = (int)((total + 7) / 8);
    const int merge_rounds = (merge_rows + 31) / 32;        // 8 workgroups x 4 rows
    const int rounds = ra.segment + merge_rounds;
    hipLaunchKernelGGL(attn_range_kernel, dim3(8 * rounds), dim3(64 * RG_WAVES), 0, stream, ra,
                       rm, merge_rounds, rounds);
    if (pl.R > 1) {
      rm = ra;
      merge_rows = p.batch * p.h_kv * ra.n_ct;
    }
  }
  if (merge_rows > 0)
    hipLaunchKernelGGL(attn_range_merge_kernel, dim3((merge_rows + 3) / 4), dim3(256), 0, stream,
                       rm);
}

static AttnArgs fast_args(const infv2_problem& p, const void* Q, const void* K, const void* V,
                          const int32_t* idx, const int32_t* n_sel, void* O, float* lse,
                          int budget, int64_t kv_cap, float scale) {
  AttnArgs a;
  a.Q = (const uint16_t*)Q;
  a.K = (const uint16_t*)K;
  a.V = (const uint16_t*)V;
  a.Kp = nullptr;
  a.Vp = nullptr;
  a.idx = idx;
  a.n_sel = n_sel;
  a.O = (uint16_t*)O;
  a.lse = lse;
  a.part_o = nullptr;
  a.part_ml = nullptr;
  a.batch = p.batch;
  a.n_q = p.n_q;
  a.q_pos0 = p.q_pos0;
  a.n_kv = p.n_kv;
  a.n_blk = (p.n_kv + AT_B - 1) / AT_B;
  a.h_kv = p.h_kv;
  a.budget = budget;
  a.kv_cap = kv_cap;
  a.c = scale * kLog2e;
  a.seq_lens = nullptr;
  a.block_table = nullptr;
  a.max_blocks = 0;
  a.n_pages = 0;
  return a;
}

// Decode of a varlen batch, optionally from a paged cache: the split kernel
// (one selected block per workgroup) and the merge; requires
// attn_use_split(p).  Workspace as attn_workspace(p, budget, true).
hipError_t launch_attn_varlen(const infv2_problem& p, const void* Q, const void* K,
                              const void* V, const int32_t* block_table, int max_blocks,
                              int n_pages, const int32_t* seq_lens, const int32_t* idx,
                              const int32_t* n_sel, void* O, float* lse, void* ws, int budget,
                              int64_t kv_cap, float scale, hipStream_t stream) {
  AttnArgs a = fast_args(p, Q, K, V, idx, n_sel, O, lse, budget, kv_cap, scale);
  a.seq_lens = seq_lens;
  a.block_table = block_table;
  a.max_blocks = max_blocks;
  a.n_pages = n_pages;
  const size_t slots = (size_t)p.batch * p.h_kv * p.n_q * budget;
  a.part_o = (float*)ws;
  a.part_ml = (float2*)((char*)ws + slots * AT_G * AT_D * sizeof(float));
  hipLaunchKernelGGL(attn_split_kernel, dim3(budget, p.h_kv, p.batch * p.n_q), dim3(64), 0,
                     stream, a);
  hipLaunchKernelGGL(attn_merge_kernel, dim3(AT_G, p.h_kv, p.batch * p.n_q), dim3(64), 0, stream,
                     a);
  return hipGetLastError();
}

// The decode step's attention with the selection's last stage inside
// (attn_split_select_kernel): the candidate lists as the selection's pool
// stage left them; writes idx and n_sel as well.  Requires attn_use_split(p)
// and one sequence length.
hipError_t launch_attn_decode_select(const infv2_problem& p, const void* Q, const void* K,
                                     const void* V, const CandLists& lists, int32_t* idx,
                                     int32_t* n_sel, void* O, float* lse, void* ws, int budget,
                                     int64_t kv_cap, float scale, hipStream_t stream) {
  AttnArgs a = fast_args(p, Q, K, V, idx, n_sel, O, lse, budget, kv_cap, scale);
  const size_t slots = (size_t)p.batch * p.h_kv * p.n_q * budget;
  a.part_o = (float*)ws;
  a.part_ml = (float2*)((char*)ws + slots * AT_G * AT_D * sizeof(float));
  DecodeSel ds;
  ds.cand = lists.cand;
  ds.idx = idx;
  ds.n_sel = n_sel;
  ds.nch = lists.nch;
  ds.kc = lists.kc;
  ds.k = p.k;
  ds.N_init = p.N_init;
  ds.N_local = p.N_local;
  hipLaunchKernelGGL(attn_split_select_kernel, dim3(budget, p.h_kv, p.batch * p.n_q), dim3(64),
                     0, stream, a, ds);
  hipLaunchKernelGGL(attn_merge_kernel, dim3(AT_G, p.h_kv, p.batch * p.n_q), dim3(64), 0, stream,
                     a);
  return hipGetLastError();
}

hipError_t launch_attn(const infv2_problem& p, const void* Q, const void* K, const void* V,
                       const int32_t* idx, const int32_t* n_sel, void* O, float* lse, void* ws,
                       int budget, int64_t kv_cap, float scale, hipStream_t stream) {
  const bool sparse = idx != nullptr;
  if (attn_fast_shape(p)) {
    AttnArgs a = fast_args(p, Q, K, V, idx, n_sel, O, lse, budget, kv_cap, scale);
    if (sparse && attn_use_split(p)) {
      const size_t slots = (size_t)p.batch * p.h_kv * p.n_q * budget;
      a.part_o = (float*)ws;
      a.part_ml = (float2*)((char*)ws + slots * AT_G * AT_D * sizeof(float));
      hipLaunchKernelGGL(attn_split_kernel, dim3(budget, p.h_kv, p.batch * p.n_q), dim3(64), 0,
                         stream, a);
      hipLaunchKernelGGL(attn_merge_kernel, dim3(AT_G, p.h_kv, p.batch * p.n_q), dim3(64), 0,
                         stream, a);
      return hipGetLastError();
    }
    const size_t pack = (size_t)p.batch * p.h_kv * a.n_blk * PACK_ELEMS;
    a.Kp = (uint16_t*)ws;
    a.Vp = (uint16_t*)ws + pack;
    hipLaunchKernelGGL(kv_pack_kernel, dim3(a.n_blk, p.h_kv, p.batch), dim3(256), 0, stream,
                       (const uint16_t*)K, (const uint16_t*)V, (uint16_t*)a.Kp, (uint16_t*)a.Vp,
                       p.n_kv, a.n_blk, p.h_kv, kv_cap);
    if (sparse) {
      const RangePlan pl = range_plan(p, budget);
      if (pl.use) {
        launch_attn_ranges(p, a, (uint16_t*)ws + 2 * pack, pl, stream);
        return hipGetLastError();
      }
    }
    const int total_qb = ((p.n_q + AT_B - 1) / AT_B) * p.batch * p.h_kv;
    dim3 grid(((total_qb + 7) / 8) * 8 * 16);
    // a list holds distinct causal blocks: at most min(budget, n_blk) entries
    if (sparse && std::min(budget, a.n_blk) > 64) {
      hipLaunchKernelGGL((attn_prefill_kernel<true, true>), grid, dim3(256), 0, stream, a);
    } else if (sparse && INFV2_ATTN_TPW > 1) {
      constexpr int TPW = INFV2_ATTN_TPW;
      const dim3 grid_seq(((total_qb + 7) / 8) * 8 * (16 / TPW));
      hipLaunchKernelGGL(attn_prefill_seq_kernel<TPW>, grid_seq, dim3(256), 0, stream, a);
    } else if (sparse) {
      hipLaunchKernelGGL((attn_prefill_kernel<true, false>), grid, dim3(256), 0, stream, a);
    } else {
      const int dn_work = ((p.n_q + DN_TOK - 1) / DN_TOK) * p.batch * p.h_kv;
      hipLaunchKernelGGL(attn_dense_kernel, dim3(((dn_work + 7) / 8) * 8), dim3(64 * DN_WAVES), 0,
                         stream, a);
    }
    return hipGetLastError();
  }
  GenericAttnArgs a;
  a.Q = Q;
  a.K = K;
  a.V = V;
  a.idx = idx;
  a.n_sel = n_sel;
  a.O = O;
  a.lse = lse;
  a.dtype = p.dtype;
  a.n_q = p.n_q;
  a.q_pos0 = p.q_pos0;
  a.n_kv = p.n_kv;
  a.h_kv = p.h_kv;
  a.G = p.G;
  a.d = p.d;
  a.B = p.B;
  a.budget = budget;
  a.kv_cap = kv_cap;
  a.scale = scale;
  dim3 grid(p.n_q, p.h_kv, p.batch);
  if (p.dtype == INFV2_F32) {
    if (sparse) hipLaunchKernelGGL((attn_generic_kernel<float, true>), grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((attn_generic_kernel<float, false>), grid, dim3(256), 0, stream, a);
  } else {
    if (sparse) hipLaunchKernelGGL((attn_generic_kernel<uint16_t, true>), grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((attn_generic_kernel<uint16_t, false>), grid, dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace infv2
