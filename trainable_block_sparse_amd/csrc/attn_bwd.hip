// Backward of the block-sparse attention (and of dense causal attention).
//
// OpenBMB blog "技术Blog-4 | 新一代InfLLM：可训练的稀疏注意力机制", 可训练稀疏注意力的
// 设计原则: the top-k selection is not differentiable and the kernels are
// parameter-free mean-pools, trained only through the token-level keys; so the
// gradients are those of the attention over the selected blocks, with the
// sets I(p) held fixed.  Per query row and head, with P the softmax of
// z = scale q.k over T(p):
//   dP_t = dO.v_t,  D = dO.O,  dZ_t = P_t (dP_t - D),
//   dq = scale sum_t dZ_t k_t,  dk_t += scale dZ_t q,  dv_t += P_t dO.
// P is recomputed from the forward's log-sum-exp.
//
// bf16 kernels (G = 16, d = 128, B = 64), fp32 gradients:
//  * bwd_pack_kernel writes, once per call, K in the key layout (the forward's
//    K pack), V in the key layout and K in the feature layout (attn_layout.hpp):
//    every MFMA operand below is one coalesced 1 KB fragment load.
//  * Sparse path (lists of at most 64 blocks): bwd_dsum_kernel writes
//    D = dO.O per (token, head); attn_bwd_dkdv_kernel (below) also stashes
//    each token's dZ for the block as a 2 KB bf16 tile in the B-operand
//    layout of dQ^T = K^T dZ^T, at the block's slot in the token's list;
//    attn_bwd_dq_stash_kernel (one wavefront per (token, group)) then reads
//    per selected block only K in the feature layout and that tile.
//  * Dense path: attn_bwd_dq_kernel, one wavefront per (token, group) as the
//    forward, recomputes S^T = K Q^T and dP^T = V dO^T (keys on the M axis,
//    the 16 heads on N), so that dZ^T lands in the B-operand layout of
//    dQ^T = K^T dZ^T; it also writes D for the dK/dV kernel.
//  * attn_bwd_dkdv_kernel: one workgroup per (key block, group, window of 2048
//    query tokens), 4 waves x 16 keys.  The tokens of the window that
//    selected the block come from a bitmap (bwd_bitmap_kernel) in ascending
//    order and are taken two at a time: S = Q K^T and dP = dO V^T with the 16
//    heads of a token on M; two permlane swaps turn P and dZ into the
//    A operand of dV = P^T dO and dK = dZ^T Q (keys on M, the 32 (token, head)
//    pairs on K), whose B operands are dO and Q transposed through LDS.  The
//    window's partial dK / dV are added to the fp32 outputs with atomics
//    (their order between windows is not fixed: the last bits of dK / dV can
//    vary between runs; dQ is deterministic).
// A generic fp64 kernel serves fp32 I/O and other shapes.
#include <algorithm>

#include "attn_layout.hpp"

namespace infv2 {

struct BwdArgs {
  const uint16_t* Q;
  const uint16_t* dO;
  const uint16_t* O;
  const float* lse;       // [b][h_q][n_q], natural log (the forward's output)
  const uint16_t* Kp;     // K, key layout
  const uint16_t* Vk;     // V, key layout
  const uint16_t* Kv;     // K, feature layout
  const int32_t* idx;     // null: dense
  const int32_t* n_sel;
  const uint32_t* bitmap; // [b][h_kv][n_blk][nw]: bit t: query token t selected the block
  float* dQ;              // [b][n_q][h_q][d]
  float* dK;              // [b][kv_cap][h_kv][d]
  float* dV;
  float* Dsum;            // [b][h_q][n_q]
  uint16_t* dZ;           // sparse: [b][h_kv][stash_tokens][budget] tiles of 2 KB (dZ of a
                          // token's selected block in the B layout of dQ^T = K^T dZ^T) for
                          // the query chunk t_base .. t_base+stash_tokens-1, or null
  int batch, n_q, q_pos0, n_kv, n_blk, h_kv, budget, nw;
  int win_base;           // first window of this dK/dV launch (the chunk's)
  int n_init, init_split; // the first n_init blocks (selected by every token) take their
                          // windows in init_split sub-windows, one workgroup each
  int t_base, t_end;      // the query chunk of this launch (dQ from the stash)
  int stash_tokens;       // query tokens the stash holds per (sequence, group)
  int64_t kv_cap;
  float c;                // scale * log2(e)
  float scale;
};

// ---------------------------------------------------------------------------
// grid: x = blocks, y = h_kv, z = batch.  256 threads.
__global__ void __launch_bounds__(256) bwd_pack_kernel(const uint16_t* __restrict__ K,
                                                       const uint16_t* __restrict__ V,
                                                       uint16_t* __restrict__ Kp,
                                                       uint16_t* __restrict__ Vk,
                                                       uint16_t* __restrict__ Kv, int n_kv,
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
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int u = tid + 256 * i;
    *(u32x4*)(Kp + base + (size_t)u * 8) = pack_piece_keys(&kt[0][0], AT_D + 8, u);
    *(u32x4*)(Vk + base + (size_t)u * 8) = pack_piece_keys(&vt[0][0], AT_D + 8, u);
    *(u32x4*)(Kv + base + (size_t)u * 8) = pack_piece_features(&kt[0][0], AT_D + 8, u);
  }
}

// n 32-bit words of zeros (dK, dV, the bitmap); grid-stride.
__global__ void __launch_bounds__(256) bwd_zero_kernel(uint32_t* __restrict__ p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256)
    p[i] = 0u;
}

// dK / dV rows 0..n_kv-1 of [b][kv_cap][row_elems] to zero.
__global__ void __launch_bounds__(256) bwd_zero_kv_kernel(float* __restrict__ dK,
                                                          float* __restrict__ dV, int n_kv,
                                                          int row_elems, int64_t kv_cap) {
  const size_t per_seq = (size_t)n_kv * row_elems;
  const int b = blockIdx.y;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < per_seq;
       i += (size_t)gridDim.x * 256) {
    const size_t off = (size_t)b * kv_cap * row_elems + i;
    dK[off] = 0.f;
    dV[off] = 0.f;
  }
}

// One thread per (sequence, group, query token): sets the token's bit in the
// row of every causal block it selected.
__global__ void __launch_bounds__(256) bwd_bitmap_kernel(BwdArgs a) {
  const size_t row = (size_t)blockIdx.x * 256 + threadIdx.x;   // (b*h_kv + g)*n_q + t
  const size_t rows = (size_t)a.batch * a.h_kv * a.n_q;
  if (row >= rows) return;
  const int t = (int)(row % a.n_q);
  const size_t bg = row / a.n_q;
  const int b_p = (a.q_pos0 + t) / AT_B;
  const int n = a.n_sel[row];
  const int32_t* sel = a.idx + row * a.budget;
  uint32_t* base = const_cast<uint32_t*>(a.bitmap) + bg * a.n_blk * a.nw + (t >> 5);
  for (int i = 0; i < n; ++i) {
    const int blk = sel[i];
    if (blk < 0 || blk > b_p) continue;
    atomicOr(base + (size_t)blk * a.nw, 1u << (t & 31));
  }
}

// D = dO . O per (token, head): one wave per (token, group), lane (grp,
// head) sums features 32ks + 8grp .. +7 (the order the dQ kernel uses), then
// the four lane groups.  grid: x = rows / 4; 256 threads.
__global__ void __launch_bounds__(256) bwd_dsum_kernel(BwdArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const size_t rid = (size_t)blockIdx.x * 4 + wave;   // (b*h_kv + g)*n_q + t
  if (rid >= (size_t)a.batch * a.h_kv * a.n_q) return;
  const int t = (int)(rid % a.n_q);
  const int bg = (int)(rid / a.n_q);
  const int g = bg % a.h_kv, b = bg / a.h_kv;
  const int grp = lane >> 4;
  const int hq = a.h_kv * AT_G;
  const int head = g * AT_G + (lane & 15);
  const size_t qoff = (((size_t)b * a.n_q + t) * hq + head) * AT_D + 8 * grp;
  float dsum = 0.f;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const u32x4 dv = *(const u32x4*)(a.dO + qoff + 32 * ks);
    const u32x4 ov = *(const u32x4*)(a.O + qoff + 32 * ks);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      dsum = __builtin_fmaf(bf16_bits_to_f32(dv[e] & 0xFFFFu), bf16_bits_to_f32(ov[e] & 0xFFFFu), dsum);
      dsum = __builtin_fmaf(bf16_bits_to_f32(dv[e] >> 16), bf16_bits_to_f32(ov[e] >> 16), dsum);
    }
  }
  dsum += __shfl_xor(dsum, 16, 64);
  dsum += __shfl_xor(dsum, 32, 64);
  if (grp == 0) a.Dsum[((size_t)b * hq + head) * a.n_q + t] = dsum;
}

// 4x4 transpose inside each quad of lanes: lane q's t[j] becomes the value
// lane j held in t[q] (two exchange stages over quad_perm DPP).
__device__ __forceinline__ void quad_transpose4(float (&t)[4], int lane) {
  const int q = lane & 3;
  float u[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float pv = __uint_as_float(dpp_u<0xB1>(__float_as_uint(t[j ^ 1])));   // lane ^ 1
    u[j] = ((j ^ q) & 1) ? pv : t[j];
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float pv = __uint_as_float(dpp_u<0x4E>(__float_as_uint(u[j ^ 2])));   // lane ^ 2
    t[j] = ((j ^ q) & 2) ? pv : u[j];
  }
}

// ---------------------------------------------------------------------------
// dQ.  Grid and token mapping as the forward prefill kernel (16 workgroups of
// 4 tokens per 64-token query block, all on one XCD).
__global__ void __launch_bounds__(256, 2) attn_bwd_dq_kernel(BwdArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n_qb = (a.n_q + AT_B - 1) / AT_B;
  const int n_bg = a.batch * a.h_kv;
  const int bid = blockIdx.x;
  const int xcd = bid & 7, r = bid >> 3;
  const int qbg = (r >> 4) * 8 + xcd;
  if (qbg >= n_qb * n_bg) return;
  const int qb = n_qb - 1 - qbg / n_bg;
  const int bg = qbg % n_bg;
  const int g = bg % a.h_kv, b = bg / a.h_kv;
  const int t = qb * AT_B + (r & 15) * 4 + wave;
  if (t >= a.n_q) return;
  const int p = a.q_pos0 + t;
  const int b_p = p / AT_B;
  const int grp = lane >> 4, r16 = lane & 15;
  const int hq = a.h_kv * AT_G;
  const int head = g * AT_G + r16;
  // B operands: Q and dO of head r16, d = 32ks + 8grp .. +7
  const size_t qoff = (((size_t)b * a.n_q + t) * hq + head) * AT_D + 8 * grp;
  bf16x8 qf[4], dof[4];
  float dsum = 0.f;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const u32x4 qv = *(const u32x4*)(a.Q + qoff + 32 * ks);
    const u32x4 dv = *(const u32x4*)(a.dO + qoff + 32 * ks);
    const u32x4 ov = *(const u32x4*)(a.O + qoff + 32 * ks);
    qf[ks] = as_bf16x8(qv);
    dof[ks] = as_bf16x8(dv);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      dsum = __builtin_fmaf(bf16_bits_to_f32(dv[e] & 0xFFFFu), bf16_bits_to_f32(ov[e] & 0xFFFFu), dsum);
      dsum = __builtin_fmaf(bf16_bits_to_f32(dv[e] >> 16), bf16_bits_to_f32(ov[e] >> 16), dsum);
    }
  }
  dsum += __shfl_xor(dsum, 16, 64);
  dsum += __shfl_xor(dsum, 32, 64);
  const float L2 = a.lse[((size_t)b * hq + head) * a.n_q + t] * kLog2e;
  if (grp == 0) a.Dsum[((size_t)b * hq + head) * a.n_q + t] = dsum;
  f32x4 acc[8];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const size_t row = ((size_t)b * a.h_kv + g) * a.n_q + t;
  const bool sparse = a.idx != nullptr;
  const int nblocks = sparse ? a.n_sel[row] : b_p + 1;
  const int32_t* sel = sparse ? a.idx + row * a.budget : nullptr;
  const size_t pack0 = ((size_t)b * a.h_kv + g) * a.n_blk * PACK_ELEMS + lane * 8;
  for (int bi = 0; bi < nblocks; ++bi) {
    const int blk = sparse ? sel[bi] : bi;
    if (blk < 0 || blk > b_p) continue;
    const size_t boff = pack0 + (size_t)blk * PACK_ELEMS;
    bf16x8 kf[4][4], vkf[4][4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        kf[tt][ks] = as_bf16x8(*(const u32x4*)(a.Kp + boff + (4 * tt + ks) * 512));
        vkf[tt][ks] = as_bf16x8(*(const u32x4*)(a.Vk + boff + (4 * tt + ks) * 512));
      }
    f32x4 s[4], dp[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      s[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
      dp[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        s[tt] = mfma16(kf[tt][ks], qf[ks], s[tt]);
        dp[tt] = mfma16(vkf[tt][ks], dof[ks], dp[tt]);
      }
    }
    bf16x8 kvf[8][2];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        kvf[mt][ks] = as_bf16x8(*(const u32x4*)(a.Kv + boff + (2 * mt + ks) * 512));
    // dZ^T = P^T (dP^T - D), keys past p masked; packed as the B operand
    // (k-step ks = keys 32ks + 8grp .. +7)
    const int kv0 = blk * AT_B;
    const bool diag = blk == b_p;
    bf16x8 dzf[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int tt = 2 * ks + (e >> 1);
        const int i0 = 2 * (e & 1);
        float z2[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int i = i0 + u;
          const int key = kv0 + tile_key(tt, 4 * grp + i);
          // masked keys take exp2(-inf) = 0: a select, no branch
          const float arg = (diag && key > p) ? kNegInf : __builtin_fmaf(s[tt][i], a.c, -L2);
          z2[u] = fast_exp2(arg) * (dp[tt][i] - dsum);
        }
        w[e] = pack_bf16x2(z2[0], z2[1]);
      }
      dzf[ks] = as_bf16x8(u32x4{w[0], w[1], w[2], w[3]});
    }
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) acc[mt] = mfma16(kvf[mt][ks], dzf[ks], acc[mt]);
  }
  // dQ^T tile mt: rows d = 16mt + 4grp + i, column = head r16
  float* drow = a.dQ + (((size_t)b * a.n_q + t) * hq + head) * AT_D;
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) {
    const f32x4 v = acc[mt] * a.scale;
    *(f32x4*)(drow + 16 * mt + 4 * grp) = v;
  }
}

// dQ from the dZ tiles the dK/dV kernel stashed (sparse path): per selected
// block only K in the feature layout (16 KB) and the 2 KB tile are read, for
// dQ^T += K^T dZ^T.  Mapping as attn_bwd_dq_kernel.  Deterministic.
__global__ void __launch_bounds__(256, 4) attn_bwd_dq_stash_kernel(BwdArgs a) {
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int qb_base = a.t_base / AT_B;                 // (t_base is a multiple of 64)
  const int n_qb = (a.t_end - a.t_base + AT_B - 1) / AT_B;
  const int n_bg = a.batch * a.h_kv;
  const int bid = blockIdx.x;
  const int xcd = bid & 7, r = bid >> 3;
  const int qbg = (r >> 4) * 8 + xcd;
  if (qbg >= n_qb * n_bg) return;
  const int qb = qb_base + n_qb - 1 - qbg / n_bg;
  const int bg = qbg % n_bg;
  const int g = bg % a.h_kv, b = bg / a.h_kv;
  const int t = qb * AT_B + (r & 15) * 4 + wave;
  if (t >= a.t_end) return;
  const int b_p = (a.q_pos0 + t) / AT_B;
  const int grp = lane >> 4, r16 = lane & 15;
  const int hq = a.h_kv * AT_G;
  f32x4 acc[8];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const size_t row = ((size_t)b * a.h_kv + g) * a.n_q + t;
  // (uniform count; the list is read into lanes 64 entries at a time, so
  // that an entry costs a lane read, not a memory round trip before its
  // block's loads)
  const int nblocks = __builtin_amdgcn_readfirstlane(a.n_sel[row]);
  const int32_t* sel = a.idx + row * a.budget;
  const size_t pack0 = ((size_t)b * a.h_kv + g) * a.n_blk * PACK_ELEMS + lane * 8;
  const size_t srow = ((size_t)b * a.h_kv + g) * a.stash_tokens + (t - a.t_base);
  const uint16_t* dz0 = a.dZ + srow * a.budget * 1024 + lane * 8;
  int list_base = 0;
  int my_entry = lane < nblocks ? sel[lane] : -1;
  for (int bi = 0; bi < nblocks; ++bi) {
    if (bi >= list_base + 64) {
      list_base = bi;
      my_entry = bi + lane < nblocks ? sel[bi + lane] : -1;
    }
    const int blk = __builtin_amdgcn_readlane(my_entry, bi - list_base);
    if (blk < 0 || blk > b_p) continue;     // never stashed
    const size_t boff = pack0 + (size_t)blk * PACK_ELEMS;
    bf16x8 kvf[8][2], dzf[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) dzf[ks] = as_bf16x8(*(const u32x4*)(dz0 + (size_t)bi * 1024 + ks * 512));
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        kvf[mt][ks] = as_bf16x8(*(const u32x4*)(a.Kv + boff + (2 * mt + ks) * 512));
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) acc[mt] = mfma16(kvf[mt][ks], dzf[ks], acc[mt]);
  }
  float* drow = a.dQ + (((size_t)b * a.n_q + t) * hq + g * AT_G + r16) * AT_D;
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) {
    const f32x4 v = acc[mt] * a.scale;
    *(f32x4*)(drow + 16 * mt + 4 * grp) = v;
  }
}

// ---------------------------------------------------------------------------
// dK, dV.  grid: x = window of BW_WIN query tokens, y = key block, z = b*h_kv.
// Tokens go two at a time (a pair) through LDS, as row-major Q and dO (the
// A operands of S = Q K^T and dP = dO V^T) and as transposed Q^T, dO^T (the
// B operands of dV = P^T dO and dK = dZ^T Q).  Wave w stages token w>>1's Q
// (w even) or dO (w odd): lane (hq = lane>>4, fo = lane&15) loads heads
// 4hq .. 4hq+3 at features 8fo .. 8fo+7 (consecutive lanes read one head's
// row), writes the four rows as they are and the transposed 8 x 4 tile as
// eight 8-byte words.  Transposed rows are 16 bytes (8 heads; two halves of
// the 16 heads) and row d sits in slot 16(d>>4) + ((d&15) ^ (d>>4)): the
// stores (rows 8 apart across lanes) and the operand reads (16 consecutive
// rows) both fall on distinct banks.  LDS holds two pairs; the registers of
// two more are in flight, so a load has two pairs of compute to land.
constexpr int BW_WIN = 2048;   // 1024: 21% slower at 32k; 4096: slower at 32k and 128k
constexpr int BW_INIT_SPLIT = 8;   // sub-windows of 256 tokens for the init blocks
constexpr int BW_RROW = AT_D + 8;   // row-major LDS row (bf16): 272 B, conflict-free reads

struct BwdTok {                      // one staged token (16 896 B)
  uint16_t R[2][AT_G][BW_RROW];      // [Q, dO][head][feature]
  uint16_t T[2][2][AT_D][8];         // [Q, dO][head half][slot of feature][8 heads]
};

__device__ __forceinline__ int bwd_tslot(int d) { return (d & ~15) | ((d & 15) ^ (d >> 4)); }

struct BwdStage {                    // one thread's share of a staged pair
  u32x4 r[4];                        // heads 4hq + j, features 8fo .. +7
  float ld;                          // L (Q waves) or D (dO waves) of head lane&15
  int32_t sel;                       // with the dZ stash: entry `lane` of the token's list
};

// STASH: also write each live token's dZ for this block to its tile in a.dZ
// (slot = the block's position in the token's list, found by a ballot over
// the list, which the staging loads bring in with Q and dO).
template <bool STASH>
__global__ void __launch_bounds__(256, 2) attn_bwd_dkdv_kernel(BwdArgs a) {
  __shared__ uint16_t toks[BW_WIN];                           // token - t_lo
  __shared__ int slot_s[2][2];                                // [buffer][token of the pair]
  __shared__ __attribute__((aligned(16))) BwdTok stg[2][2];   // [buffer][token of the pair]
  __shared__ float LD[2][2][2][AT_G];                         // [buffer][token][L, D][head]
  __shared__ int ntok_s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int win = blockIdx.x + a.win_base, bg = blockIdx.z;
  const int g = bg % a.h_kv, b = bg / a.h_kv;
  // grid y: the key blocks, then (init_split - 1) more sub-windows of each
  // init block (every token selects those, so a whole window would make one
  // long workgroup)
  int blk = blockIdx.y, sub = 0, nsub = 1;
  if (a.init_split > 1) {
    if (blk >= a.n_blk) {
      const int e = blk - a.n_blk;
      blk = e / (a.init_split - 1);
      sub = e % (a.init_split - 1) + 1;
      nsub = a.init_split;
    } else if (blk < a.n_init) {
      nsub = a.init_split;
    }
  }
  const int span = BW_WIN / nsub;                    // a multiple of 32 tokens
  const int t_lo = win * BW_WIN + sub * span;
  const int t_hi = min(min(t_lo + span, win * BW_WIN + BW_WIN), a.n_q);
  // query tokens that can see a key of the block: p >= 64 * blk
  const int t_first = max(t_lo, blk * AT_B - a.q_pos0);
  if (t_first >= t_hi) return;
  const bool sparse = a.idx != nullptr;
  if (sparse) {
    // tokens of the window that selected the block, ascending
    const int w0 = t_lo >> 5;
    const int nwin = (t_hi - t_lo + 31) >> 5;
    const uint32_t* bm = a.bitmap + ((size_t)bg * a.n_blk + blk) * a.nw + w0;
    constexpr int WPL = BW_WIN / 2048;     // bitmap words per lane of wave 0
    static_assert(WPL >= 1 && BW_WIN % 2048 == 0, "one wave scans the window's bitmap");
    if (wave == 0) {
      uint32_t word[WPL];
      int c = 0;
#pragma unroll
      for (int q = 0; q < WPL; ++q) {
        const int wi = WPL * lane + q;
        word[q] = wi < nwin ? bm[wi] : 0u;
        c += __popc(word[q]);
      }
      int incl = c;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o, 64);
        if (lane >= o) incl += y;
      }
      int pos = incl - c;
#pragma unroll
      for (int q = 0; q < WPL; ++q)
        for (uint32_t wv = word[q]; wv; wv &= wv - 1)
          toks[pos++] = (uint16_t)(32 * (WPL * lane + q) + __builtin_ctz(wv));
      if (lane == 63) ntok_s = incl;
    }
  } else {
    for (int i = tid; i < t_hi - t_first; i += 256) toks[i] = (uint16_t)(t_first - t_lo + i);
    if (tid == 0) ntok_s = t_hi - t_first;
  }
  __syncthreads();
  // (uniform: a loop bound the compiler takes as per-lane gets exec-masked
  // paths, and the wait counts of the loads in the loop become conservative)
  const int ntok = __builtin_amdgcn_readfirstlane(ntok_s);
  if (ntok == 0) return;
  const int npairs = (ntok + 1) >> 1;
  const int grp = lane >> 4, r16 = lane & 15;
  const int hq = a.h_kv * AT_G;
  // this wave's 16 keys: tile `wave` of the block (row r16 holds key
  // tile_key(wave, r16)); B operands of S = Q K^T and dP = dO V^T
  const size_t boff = (((size_t)b * a.h_kv + g) * a.n_blk + blk) * PACK_ELEMS + lane * 8;
  bf16x8 kf[4], vkf[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    kf[ks] = as_bf16x8(*(const u32x4*)(a.Kp + boff + (4 * wave + ks) * 512));
    vkf[ks] = as_bf16x8(*(const u32x4*)(a.Vk + boff + (4 * wave + ks) * 512));
  }
  const int key_l = blk * AT_B + tile_key(wave, r16);    // key of this lane's column
  // staging role: token st_k of the pair, tensor st_x (0: Q, 1: dO)
  const int st_k = wave >> 1, st_x = wave & 1;
  const int s_hq = lane >> 4, s_fo = lane & 15;
  const uint16_t* st_src = st_x ? a.dO : a.Q;
  const float* st_ld = st_x ? a.Dsum : a.lse;
  const float st_mul = st_x ? 1.f : kLog2e;
  // Branch-free loads (a branch around them would make the compiler wait for
  // them at its end): a missing second token of the last pair stages the
  // window's first token instead, whose finite values its masked P and dZ
  // (exact zeros) then cancel.
  auto stage_load = [&](int pair, BwdStage& s) {
    const int k = 2 * pair + st_k;
    const int tt = t_lo + toks[k < ntok ? k : 0];
    const size_t off = (((size_t)b * a.n_q + tt) * hq + g * AT_G + 4 * s_hq) * AT_D + 8 * s_fo;
#pragma unroll
    for (int j = 0; j < 4; ++j) s.r[j] = *(const u32x4*)(st_src + off + j * AT_D);
    s.ld = st_ld[((size_t)b * hq + g * AT_G + (lane & 15)) * a.n_q + tt];
    if constexpr (STASH)
      s.sel = a.idx[(((size_t)b * a.h_kv + g) * a.n_q + tt) * a.budget + min(lane, a.budget - 1)];
  };
  auto stage_store = [&](int buf, const BwdStage& s) {
    BwdTok& T = stg[buf][st_k];
#pragma unroll
    for (int j = 0; j < 4; ++j) *(u32x4*)&T.R[st_x][4 * s_hq + j][8 * s_fo] = s.r[j];
    uint16_t* th = &T.T[st_x][s_hq >> 1][0][4 * (s_hq & 1)];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      // features 8fo + 2m (low halves) and 8fo + 2m + 1 (high halves), heads 4hq .. +3
      const u32x2 lo = {(s.r[0][m] & 0xFFFFu) | (s.r[1][m] << 16),
                        (s.r[2][m] & 0xFFFFu) | (s.r[3][m] << 16)};
      const u32x2 hi = {(s.r[0][m] >> 16) | (s.r[1][m] & 0xFFFF0000u),
                        (s.r[2][m] >> 16) | (s.r[3][m] & 0xFFFF0000u)};
      *(u32x2*)(th + 8 * bwd_tslot(8 * s_fo + 2 * m)) = lo;
      *(u32x2*)(th + 8 * bwd_tslot(8 * s_fo + 2 * m + 1)) = hi;
    }
    // lanes l, l+16, l+32, l+48 hold the same value: all write it, with no
    // branch (a branch would wait for every load in flight)
    LD[buf][st_k][st_x][lane & 15] = s.ld * st_mul;
    if constexpr (STASH) {
      const uint64_t hit = __ballot(lane < a.budget && s.sel == blk);
      if (st_x == 0 && lane == 0) slot_s[buf][st_k] = hit ? (int)__builtin_ctzll(hit) : -1;
    }
  };
  f32x4 accV[8], accK[8];
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) {
    accV[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    accK[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  auto compute = [&](int buf, int pair) {
    const int tA = t_lo + toks[2 * pair];
    const int tB = 2 * pair + 1 < ntok ? t_lo + toks[2 * pair + 1] : -1;
    // the (token, head) normalisers and D of this lane's rows
    float Lr[2][4], Dr[2][4];
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        Lr[k2][j] = LD[buf][k2][0][4 * grp + j];
        Dr[k2][j] = LD[buf][k2][1][4 * grp + j];
      }
    // S and dP for both tokens: rows = heads 4grp + j, column = key key_l
    f32x4 sc[2], dpv[2];
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      sc[k2] = f32x4{0.f, 0.f, 0.f, 0.f};
      dpv[k2] = f32x4{0.f, 0.f, 0.f, 0.f};
      const BwdTok& T = stg[buf][k2];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 qa = as_bf16x8(*(const u32x4*)&T.R[0][r16][32 * ks + 8 * grp]);
        const bf16x8 da = as_bf16x8(*(const u32x4*)&T.R[1][r16][32 * ks + 8 * grp]);
        sc[k2] = mfma16(qa, kf[ks], sc[k2]);
        dpv[k2] = mfma16(da, vkf[ks], dpv[k2]);
      }
    }
    // P and dZ (0 for masked keys and for a missing second token)
    f32x4 pv[2], zv[2];
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
      const int tt = k2 == 0 ? tA : tB;
      const bool live = tt >= 0 && key_l <= a.q_pos0 + tt;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // masked entries take exp2(-inf) = 0: a select, no branch
        const float arg = live ? __builtin_fmaf(sc[k2][j], a.c, -Lr[k2][j]) : kNegInf;
        const float pr = fast_exp2(arg);
        pv[k2][j] = pr;
        zv[k2][j] = pr * (dpv[k2][j] - Dr[k2][j]);
      }
    }
    // to A operands: lane row r16 = key, k = 8*grp + e = the 32 (token, head)
    // pairs (grp 0, 1: token A heads 0-7, 8-15; grp 2, 3: token B)
    bf16x8 pa, za;
    {
      float xp[4], yp[4], xz[4], yz[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const auto s1 = __builtin_amdgcn_permlane32_swap(__float_as_uint(pv[0][j]),
                                                         __float_as_uint(pv[1][j]), false, false);
        const auto s2 = __builtin_amdgcn_permlane16_swap(s1[0], s1[1], false, false);
        xp[j] = __uint_as_float(s2[0]);
        yp[j] = __uint_as_float(s2[1]);
        const auto z1 = __builtin_amdgcn_permlane32_swap(__float_as_uint(zv[0][j]),
                                                         __float_as_uint(zv[1][j]), false, false);
        const auto z2 = __builtin_amdgcn_permlane16_swap(z1[0], z1[1], false, false);
        xz[j] = __uint_as_float(z2[0]);
        yz[j] = __uint_as_float(z2[1]);
      }
      pa = as_bf16x8(u32x4{pack_bf16x2(xp[0], xp[1]), pack_bf16x2(xp[2], xp[3]),
                           pack_bf16x2(yp[0], yp[1]), pack_bf16x2(yp[2], yp[3])});
      za = as_bf16x8(u32x4{pack_bf16x2(xz[0], xz[1]), pack_bf16x2(xz[2], xz[3]),
                           pack_bf16x2(yz[0], yz[1]), pack_bf16x2(yz[2], yz[3])});
    }
    // dV += P^T dO, dK += dZ^T Q: B operand lane = feature 16nt + r16,
    // k = the 8 heads 8(grp&1) .. of token grp>>1
    const BwdTok& T = stg[buf][grp >> 1];
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      const int slot = 16 * nt + (r16 ^ nt);
      const bf16x8 bq = as_bf16x8(*(const u32x4*)&T.T[0][grp & 1][slot][0]);
      const bf16x8 bd = as_bf16x8(*(const u32x4*)&T.T[1][grp & 1][slot][0]);
      accV[nt] = mfma16(pa, bd, accV[nt]);
      accK[nt] = mfma16(za, bq, accK[nt]);
    }
    // (after the MFMAs are issued, so that this vector work overlaps them)
    if constexpr (STASH) {
      // dZ of the wave's 16 keys (key 32ks + 8m + 4(wave&1) + q sits in lane
      // row r16 = 4m + q, ks = wave>>1) to the token's tile: after a
      // transpose inside each quad, lane (grp, 4m + q') holds head 4grp + q'
      // at the four keys q = 0..3 -- 8 bytes of the tile's 16-byte piece
      // (ks, lane 16m + head), elements 4(wave&1) .. +3
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        float tz[4] = {zv[k2][0], zv[k2][1], zv[k2][2], zv[k2][3]};
        quad_transpose4(tz, lane);
        const int tt = k2 == 0 ? tA : tB;
        const int slot = slot_s[buf][k2];
        if (tt >= 0 && slot >= 0) {
          const size_t trow = ((size_t)b * a.h_kv + g) * a.stash_tokens + (tt - a.t_base);
          const int piece = (wave >> 1) * 64 + 16 * (r16 >> 2) + 4 * grp + (lane & 3);
          *(u32x2*)(a.dZ + ((trow * a.budget + slot) * 128 + piece) * 8 + 4 * (wave & 1)) =
              u32x2{pack_bf16x2(tz[0], tz[1]), pack_bf16x2(tz[2], tz[3])};
        }
      }
    }
  };
  // pipeline: pair i is read from buffer i&1; set A holds the registers of
  // even pairs, set B of odd pairs, loaded two pairs ahead.  Loads and stores
  // are unconditional (pair indices past the end are clamped to the last
  // pair, whose copies are never read): a load under a branch would make the
  // compiler wait for all loads in flight where the branch joins.  For the
  // same reason the loop has no exit between its two halves (an odd last
  // pair is computed after it) and the first loads are issued in the loop's
  // order (the scheduling barriers keep them so).
  const int last = npairs - 1;
  BwdStage sa, sb;
  stage_load(0, sa);
  __builtin_amdgcn_sched_barrier(0);
  stage_load(min(1, last), sb);
  __builtin_amdgcn_sched_barrier(0);
  stage_store(0, sa);
  __builtin_amdgcn_sched_barrier(0);
  stage_load(min(2, last), sa);
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();
  int i = 0;
  for (; i + 1 < npairs; i += 2) {
    compute(0, i);
    stage_store(1, sb);
    stage_load(min(i + 3, last), sb);
    __syncthreads();
    compute(1, i + 1);
    stage_store(0, sa);
    stage_load(min(i + 4, last), sa);
    __syncthreads();
  }
  if (i < npairs) compute(0, i);
  // C layout: rows = keys tile_key(wave, 4grp + j), column = feature 16nt + r16
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int key = blk * AT_B + tile_key(wave, 4 * grp + j);
    if (key >= a.n_kv) continue;
    const size_t off = (((size_t)b * a.kv_cap + key) * a.h_kv + g) * AT_D + r16;
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      atomicAdd(a.dV + off + 16 * nt, accV[nt][j]);
      atomicAdd(a.dK + off + 16 * nt, accK[nt][j] * a.scale);
    }
  }
}

// ---------------------------------------------------------------------------
// Generic shapes (fp32 I/O, other G, d, B): one workgroup per (token, group),
// fp64 math; dK / dV by fp32 atomics.  Dynamic LDS: 2 * max keys doubles.
struct GenericBwdArgs {
  const void* Q;
  const void* K;
  const void* V;
  const void* O;
  const void* dO;
  const float* lse;
  const int32_t* idx;
  const int32_t* n_sel;
  float* dQ;
  float* dK;
  float* dV;
  int n_q, q_pos0, n_kv, h_kv, G, d, B, budget, max_keys;
  int64_t kv_cap;
  double scale;
};

template <typename T> __device__ __forceinline__ double bld(const T* p, size_t i);
template <> __device__ __forceinline__ double bld<float>(const float* p, size_t i) { return p[i]; }
template <> __device__ __forceinline__ double bld<uint16_t>(const uint16_t* p, size_t i) {
  return (double)bf16_bits_to_f32(p[i]);
}

__device__ double bwd_block_sum(double v, double* red) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  double r = 0.0;
  for (int i = 0; i < nw; ++i) r += red[i];
  return r;
}

template <typename T, bool SPARSE>
__global__ void __launch_bounds__(256) attn_bwd_generic_kernel(GenericBwdArgs a) {
  extern __shared__ double gdyn[];
  __shared__ double red[8];
  __shared__ int keys_s[1];
  double* pz = gdyn;                 // [max_keys]: P_t, then dZ_t
  double* pp = gdyn + a.max_keys;    // [max_keys]: P_t
  int* klist = (int*)(gdyn + 2 * (size_t)a.max_keys);   // [max_keys] key positions
  const int t = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int p = a.q_pos0 + t;
  const int b_p = p / a.B;
  const int hq = a.h_kv * a.G;
  const T* Q = (const T*)a.Q;
  const T* K = (const T*)a.K;
  const T* V = (const T*)a.V;
  const T* O = (const T*)a.O;
  const T* dO = (const T*)a.dO;
  // the attended keys T(p), ascending
  if (threadIdx.x == 0) {
    int n = 0;
    const size_t row = ((size_t)b * a.h_kv + g) * a.n_q + t;
    const int nb = SPARSE ? a.n_sel[row] : b_p + 1;
    for (int i = 0; i < nb; ++i) {
      const int blk = SPARSE ? a.idx[row * a.budget + i] : i;
      if (blk < 0 || blk > b_p) continue;
      for (int key = blk * a.B; key < min(blk * a.B + a.B, p + 1); ++key) klist[n++] = key;
    }
    keys_s[0] = n;
  }
  __syncthreads();
  const int nk = keys_s[0];
  for (int hh = 0; hh < a.G; ++hh) {
    const int h = g * a.G + hh;
    const size_t qo = (((size_t)b * a.n_q + t) * hq + h) * a.d;
    const double L = (double)a.lse[((size_t)b * hq + h) * a.n_q + t];
    // D = dO . O
    double dpart = 0.0;
    for (int i = threadIdx.x; i < a.d; i += blockDim.x) dpart += bld<T>(dO, qo + i) * bld<T>(O, qo + i);
    const double D = bwd_block_sum(dpart, red);
    for (int j = threadIdx.x; j < nk; j += blockDim.x) {
      const size_t ko = (((size_t)b * a.kv_cap + klist[j]) * a.h_kv + g) * a.d;
      double z = 0.0, dp = 0.0;
      for (int i = 0; i < a.d; ++i) {
        z += bld<T>(Q, qo + i) * bld<T>(K, ko + i);
        dp += bld<T>(dO, qo + i) * bld<T>(V, ko + i);
      }
      const double pr = exp(z * a.scale - L);
      pp[j] = pr;
      pz[j] = pr * (dp - D);
    }
    __syncthreads();
    for (int i = threadIdx.x; i < a.d; i += blockDim.x) {
      double acc = 0.0;
      for (int j = 0; j < nk; ++j)
        acc += pz[j] * bld<T>(K, (((size_t)b * a.kv_cap + klist[j]) * a.h_kv + g) * a.d + i);
      a.dQ[qo + i] = (float)(acc * a.scale);
    }
    for (size_t u = threadIdx.x; u < (size_t)nk * a.d; u += blockDim.x) {
      const int j = (int)(u / a.d), i = (int)(u % a.d);
      const size_t ko = (((size_t)b * a.kv_cap + klist[j]) * a.h_kv + g) * a.d + i;
      atomicAdd(a.dK + ko, (float)(pz[j] * a.scale * bld<T>(Q, qo + i)));
      atomicAdd(a.dV + ko, (float)(pp[j] * bld<T>(dO, qo + i)));
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
bool attn_fast_shape(const infv2_problem& p);

static size_t bwd_nw(const infv2_problem& p) { return ((size_t)p.n_q + 31) / 32; }

// The sparse path stashes dZ (2 KB per selected block of every row) when a
// row's list fits one wave's ballot.
static bool bwd_stash(const infv2_problem& p, bool sparse) {
  return sparse && p.N_init + p.N_local + p.k <= 64;
}
// Workspace apart from the dZ stash: K/V packs, the dO.O row sums and the
// sparse path's block-to-query bitmap.
static size_t bwd_fixed_bytes(const infv2_problem& p, bool sparse) {
  const size_t n_blk = ((size_t)p.n_kv + AT_B - 1) / AT_B;
  const size_t packs = 3 * (size_t)p.batch * p.h_kv * n_blk * PACK_ELEMS * sizeof(uint16_t);
  const size_t dsum = (size_t)p.batch * p.h_kv * AT_G * p.n_q * sizeof(float);
  const size_t bitmap = sparse ? (size_t)p.batch * p.h_kv * n_blk * bwd_nw(p) * sizeof(uint32_t) : 0;
  return packs + ((dsum + 255) & ~(size_t)255) + ((bitmap + 255) & ~(size_t)255);
}
// The stash holds a chunk of whole BW_WIN-token windows of queries, as many
// as keep the whole workspace within BWD_WS_BUDGET bytes (at least one
// window); the backward runs chunk by chunk (dK/dV with the stash, then dQ
// from it).
constexpr size_t BWD_WS_BUDGET = (size_t)1 << 30;
static int bwd_stash_tokens(const infv2_problem& p) {
  const size_t per_tok = (size_t)p.batch * p.h_kv * (p.N_init + p.N_local + p.k) * 2048;
  const size_t fixed = bwd_fixed_bytes(p, true);
  const size_t room = fixed < BWD_WS_BUDGET ? BWD_WS_BUDGET - fixed : 0;
  const size_t fit = room / per_tok / BW_WIN * BW_WIN;
  const size_t chunk = fit < (size_t)BW_WIN ? (size_t)BW_WIN : fit;
  return (int)(chunk < (size_t)p.n_q ? chunk : (size_t)p.n_q);
}

size_t attn_bwd_workspace(const infv2_problem& p, bool sparse) {
  if (!attn_fast_shape(p)) return 0;
  const size_t dz = bwd_stash(p, sparse) ? (size_t)p.batch * p.h_kv * bwd_stash_tokens(p) *
                                               (p.N_init + p.N_local + p.k) * 2048
                                         : 0;
  return bwd_fixed_bytes(p, sparse) + dz;
}

size_t attn_bwd_generic_lds(const infv2_problem& p, int budget, bool sparse) {
  const size_t max_keys = sparse ? (size_t)budget * p.B : (size_t)p.n_kv;
  return max_keys * (2 * sizeof(double) + sizeof(int));
}

hipError_t launch_attn_bwd(const infv2_problem& p, const void* Q, const void* K, const void* V,
                           const int32_t* idx, const int32_t* n_sel, const void* O,
                           const float* lse, const void* dO, float* dQ, float* dK, float* dV,
                           void* ws, int budget, int64_t kv_cap, float scale,
                           hipStream_t stream) {
  const bool sparse = idx != nullptr;
  const int n_blk = (p.n_kv + AT_B - 1) / AT_B;
  {  // dK, dV rows 0..n_kv-1 start at zero
    const size_t per_seq = (size_t)p.n_kv * p.h_kv * p.d;
    const size_t blocks = (per_seq + 255) / 256;
    const int gx = (int)(blocks < 4096 ? blocks : 4096);
    hipLaunchKernelGGL(bwd_zero_kv_kernel, dim3(gx, p.batch), dim3(256), 0, stream, dK, dV,
                       p.n_kv, p.h_kv * p.d, kv_cap);
  }
  if (attn_fast_shape(p)) {
    BwdArgs a = {};
    a.Q = (const uint16_t*)Q;
    a.dO = (const uint16_t*)dO;
    a.O = (const uint16_t*)O;
    a.lse = lse;
    const size_t pack = (size_t)p.batch * p.h_kv * n_blk * PACK_ELEMS;
    a.Kp = (const uint16_t*)ws;
    a.Vk = (const uint16_t*)ws + pack;
    a.Kv = (const uint16_t*)ws + 2 * pack;
    char* tail = (char*)ws + 3 * pack * sizeof(uint16_t);
    a.Dsum = (float*)tail;
    const size_t dsum = (size_t)p.batch * p.h_kv * AT_G * p.n_q * sizeof(float);
    a.bitmap = sparse ? (const uint32_t*)(tail + ((dsum + 255) & ~(size_t)255)) : nullptr;
    const size_t bitmap_bytes = sparse ? (size_t)p.batch * p.h_kv * n_blk * bwd_nw(p) * sizeof(uint32_t) : 0;
    a.dZ = bwd_stash(p, sparse) ? (uint16_t*)(tail + ((dsum + 255) & ~(size_t)255) +
                                              ((bitmap_bytes + 255) & ~(size_t)255))
                                : nullptr;
    a.idx = idx;
    a.n_sel = n_sel;
    a.dQ = dQ;
    a.dK = dK;
    a.dV = dV;
    a.batch = p.batch;
    a.n_q = p.n_q;
    a.q_pos0 = p.q_pos0;
    a.n_kv = p.n_kv;
    a.n_blk = n_blk;
    a.h_kv = p.h_kv;
    a.budget = budget;
    a.nw = (int)bwd_nw(p);
    a.kv_cap = kv_cap;
    a.c = scale * kLog2e;
    a.scale = scale;
    hipLaunchKernelGGL(bwd_pack_kernel, dim3(n_blk, p.h_kv, p.batch), dim3(256), 0, stream,
                       (const uint16_t*)K, (const uint16_t*)V, (uint16_t*)a.Kp, (uint16_t*)a.Vk,
                       (uint16_t*)a.Kv, p.n_kv, n_blk, p.h_kv, kv_cap);
    if (sparse) {
      const size_t words = (size_t)p.batch * p.h_kv * n_blk * a.nw;
      const size_t zblocks = (words + 255) / 256;
      const int gz = (int)(zblocks < 4096 ? zblocks : 4096);
      hipLaunchKernelGGL(bwd_zero_kernel, dim3(gz), dim3(256), 0, stream,
                         const_cast<uint32_t*>(a.bitmap), words);
      const size_t rows = (size_t)p.batch * p.h_kv * p.n_q;
      hipLaunchKernelGGL(bwd_bitmap_kernel, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0,
                         stream, a);
    }
    const int total_qb = ((p.n_q + AT_B - 1) / AT_B) * p.batch * p.h_kv;
    const dim3 dq_grid(((total_qb + 7) / 8) * 8 * 16);
    const dim3 kv_grid((p.n_q + BW_WIN - 1) / BW_WIN, n_blk, p.batch * p.h_kv);
    if (a.dZ) {
      // D first, then per query chunk: dK/dV (which stashes dZ), then dQ
      // from the stash
      const size_t rows = (size_t)p.batch * p.h_kv * p.n_q;
      hipLaunchKernelGGL(bwd_dsum_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream, a);
      a.stash_tokens = bwd_stash_tokens(p);
      a.n_init = std::min(p.N_init, n_blk);
      a.init_split = BW_INIT_SPLIT;
      for (int t0 = 0; t0 < p.n_q; t0 += a.stash_tokens) {
        a.t_base = t0;
        a.t_end = std::min(p.n_q, t0 + a.stash_tokens);
        a.win_base = t0 / BW_WIN;
        const int n_win = (a.t_end - t0 + BW_WIN - 1) / BW_WIN;
        const int chunk_qb = ((a.t_end - t0 + AT_B - 1) / AT_B) * p.batch * p.h_kv;
        hipLaunchKernelGGL(attn_bwd_dkdv_kernel<true>,
                           dim3(n_win, n_blk + a.n_init * (BW_INIT_SPLIT - 1), p.batch * p.h_kv),
                           dim3(256), 0, stream, a);
        hipLaunchKernelGGL(attn_bwd_dq_stash_kernel, dim3(((chunk_qb + 7) / 8) * 8 * 16),
                           dim3(256), 0, stream, a);
      }
    } else {
      hipLaunchKernelGGL(attn_bwd_dq_kernel, dq_grid, dim3(256), 0, stream, a);
      hipLaunchKernelGGL(attn_bwd_dkdv_kernel<false>, kv_grid, dim3(256), 0, stream, a);
    }
    return hipGetLastError();
  }
  GenericBwdArgs a = {};
  a.Q = Q;
  a.K = K;
  a.V = V;
  a.O = O;
  a.dO = dO;
  a.lse = lse;
  a.idx = idx;
  a.n_sel = n_sel;
  a.dQ = dQ;
  a.dK = dK;
  a.dV = dV;
  a.n_q = p.n_q;
  a.q_pos0 = p.q_pos0;
  a.n_kv = p.n_kv;
  a.h_kv = p.h_kv;
  a.G = p.G;
  a.d = p.d;
  a.B = p.B;
  a.budget = budget;
  a.max_keys = sparse ? budget * p.B : p.n_kv;
  a.kv_cap = kv_cap;
  a.scale = scale;
  const size_t lds = attn_bwd_generic_lds(p, budget, sparse);
  dim3 grid(p.n_q, p.h_kv, p.batch);
  if (p.dtype == INFV2_F32) {
    if (sparse) hipLaunchKernelGGL((attn_bwd_generic_kernel<float, true>), grid, dim3(256), lds, stream, a);
    else hipLaunchKernelGGL((attn_bwd_generic_kernel<float, false>), grid, dim3(256), lds, stream, a);
  } else {
    if (sparse) hipLaunchKernelGGL((attn_bwd_generic_kernel<uint16_t, true>), grid, dim3(256), lds, stream, a);
    else hipLaunchKernelGGL((attn_bwd_generic_kernel<uint16_t, false>), grid, dim3(256), lds, stream, a);
  }
  return hipGetLastError();
}

}  // namespace infv2
