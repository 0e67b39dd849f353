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
#include "attn_layout.hpp"

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
// LONG: block lists of more than 64 entries (budget > 64) are re-read 64 at a
// time; the common case never touches memory for the list inside the loop.
template <bool SPARSE, bool LONG>
__global__ void __launch_bounds__(256, 1) attn_prefill_kernel(AttnArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
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
  const int nblocks = SPARSE ? a.n_sel[row] : b_p + 1;
  const int32_t* sel = SPARSE ? a.idx + row * a.budget : nullptr;
  const size_t pack0 = ((size_t)b * a.h_kv + g) * a.n_blk * PACK_ELEMS + lane * 8;
  const uint16_t* kbase = a.Kp + pack0;
  const uint16_t* vbase = a.Vp + pack0;
  const int grp = lane >> 4, r16 = lane & 15;
  // The block list is held one entry per lane, 64 entries at a time, so that
  // reading the next entry (a uniform lane read) never waits on memory.
  int list_base = 0;
  int my_entry = (SPARSE && lane < nblocks) ? sel[lane] : -1;
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
  // Every iteration issues the loads of the next entry unconditionally (the
  // last one re-reads its own block), so the loads in flight are the same on
  // every path and the waits stay precise.  A non-causal entry is processed as
  // block 0 with every key masked: it adds nothing.
  // Two register sets (A: even list entries, B: odd ones): the K and V of
  // entries i+1 and i+2 are in flight while entry i is computed.
  bf16x8 kA[4][4], vA[8][2], kB[4][4], vB[8][2], pf[2];
  auto step = [&](int blk, bf16x8 (&kf)[4][4], bf16x8 (&vf)[8][2], int nxt) {
    const int kv0 = max(blk, 0) * AT_B;
    if (blk == b_p)
      attn_scores<true>(qf, kf, o, m_run, l_run, kv0, p, a.c, lane, pf);
    else if (blk < 0)
      attn_scores<true>(qf, kf, o, m_run, l_run, kv0, -1, a.c, lane, pf);
    else
      attn_scores<false>(qf, kf, o, m_run, l_run, kv0, p, a.c, lane, pf);
    load_k(max(nxt, 0), kf);
    __builtin_amdgcn_sched_barrier(0);
    attn_pv(vf, pf, o);
    load_v(max(nxt, 0), vf);
    __builtin_amdgcn_sched_barrier(0);
  };
  int b0 = block_at(0);
  int b1 = block_at(min(1, nblocks - 1));
  load_k(max(b0, 0), kA);
  load_v(max(b0, 0), vA);
  load_k(max(b1, 0), kB);
  load_v(max(b1, 0), vB);
  for (int bi = 0; bi < nblocks; bi += 2) {
    const int n2 = block_at(min(bi + 2, nblocks - 1));
    step(b0, kA, vA, n2);
    if (bi + 1 >= nblocks) break;
    const int n3 = block_at(min(bi + 3, nblocks - 1));
    step(b1, kB, vB, n3);
    b0 = n2;
    b1 = n3;
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

__global__ void __launch_bounds__(64) attn_split_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t kst[AT_B * AT_D * 2];
  __shared__ __attribute__((aligned(16))) uint16_t vt2[8][AT_D][8];
  const int lane = threadIdx.x;
  const int slot = blockIdx.x, g = blockIdx.y, bt = blockIdx.z;
  const int b = bt / a.n_q, t = bt % a.n_q;
  const size_t row = ((size_t)b * a.h_kv + g) * a.n_q + t;
  const size_t prow = row * a.budget + slot;
  const int nsel = a.n_sel[row];
  if (slot >= nsel) return;
  const int n_kv = a.seq_lens ? seq_len_of(a.seq_lens, b, a.n_q, a.n_kv) : a.n_kv;
  const int p = (a.seq_lens ? n_kv - a.n_q : a.q_pos0) + t;
  const int blk = a.idx[row * a.budget + slot];
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
  bf16x8 qf[4];
  load_qfrag(a, b, t, g, lane, qf);
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

size_t attn_workspace(const infv2_problem& p, int budget, bool sparse) {
  if (!attn_fast_shape(p)) return 0;
  if (sparse && attn_use_split(p)) {
    const size_t slots = (size_t)p.batch * p.h_kv * p.n_q * budget;
    return slots * AT_G * AT_D * sizeof(float) + slots * AT_G * sizeof(float2);
  }
  const size_t n_blk = ((size_t)p.n_kv + AT_B - 1) / AT_B;
  return 2 * (size_t)p.batch * p.h_kv * n_blk * PACK_ELEMS * sizeof(uint16_t);
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
    const int total_qb = ((p.n_q + AT_B - 1) / AT_B) * p.batch * p.h_kv;
    dim3 grid(((total_qb + 7) / 8) * 8 * 16);
    if (sparse && budget > 64) {
      hipLaunchKernelGGL((attn_prefill_kernel<true, true>), grid, dim3(256), 0, stream, a);
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
