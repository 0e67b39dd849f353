// Stage 1 of the block representation: mean-pooled keys K^C1.
//
// papernotes.org InfLLM-V2 note, 方法详解 > 关键设计 3 (three-stage compression,
// stage 1 with kernel length l_C1 and stride s_C1); OpenBMB blog
// "技术Blog-4 | 新一代InfLLM：可训练的稀疏注意力机制", 动态上下文块选择 > 语义核 (kernels
// overlap, keys only, representation = mean of the kernel's keys).
//
// The kernel is HBM-bound: every key row is read by l_C1/s_C1 kernels, so the
// second read hits L2.  Threads run along d so that each 32-token segment is
// read as contiguous rows.  The exact mean and its single rounding are in
// kc1_mean.hpp (shared with the decode logits kernel's on-the-fly append).
#include "kc1_mean.hpp"

namespace infv2 {

template <typename T> __device__ __forceinline__ double load_f64(const T* p);
template <> __device__ __forceinline__ double load_f64<uint16_t>(const uint16_t* p) {
  return (double)bf16_bits_to_f32(*p);
}
template <> __device__ __forceinline__ double load_f64<float>(const float* p) {
  return (double)*p;
}

template <typename T> __device__ __forceinline__ void store_rounded(T* p, double hi, double lo);
template <> __device__ __forceinline__ void store_rounded<uint16_t>(uint16_t* p, double hi, double lo) {
  *p = kmean_bf16(hi, lo);
}
template <> __device__ __forceinline__ void store_rounded<float>(float* p, double hi, double lo) {
  *p = (float)round_pair<24>(hi, lo);                 // exact conversion
}

// Where the keys come from.  Contiguous: K [b][kv_cap][h_kv][d], kernels
// [c1_begin, c1_end) of every sequence.  Varlen (seq_lens set): sequence b
// holds seq_lens[b] keys (clamped to [n_q, n_kv]) and gets its last `last_n`
// complete kernels (all of them when last_n <= 0), c1_begin/c1_end unused.
// Paged (block_table set): K is a pool of n_pages pages [B][h_kv][d], token
// u of sequence b in page block_table[b * max_blocks + u / B] (clamped into
// the pool).
struct CompressSrc {
  const int32_t* seq_lens;
  const int32_t* block_table;
  int max_blocks, n_pages, B, n_q, n_kv, last_n;
};

// grid: x = kernel groups of (blockDim / d) kernels, y = h_kv, z = batch.
template <typename T>
__global__ void __launch_bounds__(256) compress_k_kernel(
    const T* __restrict__ K, T* __restrict__ Kc1, int c1_begin, int c1_end, int h_kv, int d,
    int64_t kv_cap, int64_t c1_cap, int l_C1, int s_C1, double inv_l, CompressSrc src_of) {
  const int per_blk = blockDim.x / d;
  const int local = threadIdx.x / d;
  const int di = threadIdx.x % d;
  if (local >= per_blk) return;
  const int g = blockIdx.y, b = blockIdx.z;
  int j_lo = c1_begin, j_hi = c1_end;
  if (src_of.seq_lens) {
    const int len = seq_len_of(src_of.seq_lens, b, src_of.n_q, src_of.n_kv);
    j_hi = len < l_C1 ? 0 : (len - l_C1) / s_C1 + 1;
    j_lo = src_of.last_n > 0 ? max(0, j_hi - src_of.last_n) : 0;
  }
  const int j = j_lo + blockIdx.x * per_blk + local;
  if (j >= j_hi) return;
  const size_t row_stride = (size_t)h_kv * d;
  const size_t col = (size_t)g * d + di;
  const T* seq_base = K + (size_t)b * kv_cap * row_stride + col;
  const int32_t* table = src_of.block_table ? src_of.block_table + (size_t)b * src_of.max_blocks
                                            : nullptr;
  double hi = 0.0, lo = 0.0;
  // 32 keys per step, all loaded before the (serial) compensated sum
  for (int u0 = 0; u0 < l_C1; u0 += 32) {
    const int cnt = min(32, l_C1 - u0);
    double x[32];
    // paged: the group's 32 tokens lie in at most two pages (B >= 32 on
    // this path), looked up once each before the loads
    const int tok0 = j * s_C1 + u0;
    int pg0 = 0, pg1 = 0;
    if (table) {
      pg0 = min(max(table[tok0 / src_of.B], 0), src_of.n_pages - 1);
      pg1 = min(max(table[(tok0 + cnt - 1) / src_of.B], 0), src_of.n_pages - 1);
    }
#pragma unroll
    for (int u = 0; u < 32; ++u) {
      const int tok = tok0 + min(u, cnt - 1);
      size_t row = tok;   // token row of the sequence, or of its page in the pool
      if (table)
        row = (size_t)(tok / src_of.B == tok0 / src_of.B ? pg0 : pg1) * src_of.B + tok % src_of.B;
      x[u] = load_f64<T>((table ? K + col : seq_base) + row * row_stride);
    }
#pragma unroll
    for (int u = 0; u < 32; ++u) {
      // (a predicate, not a break: the unrolled loop keeps x in registers;
      // -0 is the exact identity of +)
      kmean_add(hi, lo, u < cnt ? x[u] : -0.0);
    }
  }
  double rh, rl;
  kmean_finish(hi, lo, inv_l, rh, rl);
  T* dst = Kc1 + (((size_t)b * h_kv + g) * c1_cap + j) * d + di;
  store_rounded<T>(dst, rh, rl);
}

// Kernels of length l_len at stride s_len (K^C1: l_C1, s_C1; K^C2: 4 l_C1, 4 s_C1).
hipError_t launch_compress_k(const infv2_problem& p, const void* K, void* Kc1, int c1_begin,
                             int c1_end, int64_t kv_cap, int64_t c1_cap, int l_len, int s_len,
                             hipStream_t stream) {
  if (c1_end <= c1_begin) return hipSuccess;
  const int per_blk = 256 / p.d;
  const int n = c1_end - c1_begin;
  dim3 grid((n + per_blk - 1) / per_blk, p.h_kv, p.batch);
  dim3 block(per_blk * p.d);
  const double inv_l = 1.0 / (double)l_len;
  const CompressSrc src = {nullptr, nullptr, 0, 0, p.B, p.n_q, p.n_kv, 0};
  if (p.dtype == INFV2_BF16) {
    hipLaunchKernelGGL(compress_k_kernel<uint16_t>, grid, block, 0, stream,
                       (const uint16_t*)K, (uint16_t*)Kc1, c1_begin, c1_end, p.h_kv, p.d, kv_cap,
                       c1_cap, l_len, s_len, inv_l, src);
  } else {
    hipLaunchKernelGGL(compress_k_kernel<float>, grid, block, 0, stream, (const float*)K,
                       (float*)Kc1, c1_begin, c1_end, p.h_kv, p.d, kv_cap, c1_cap, l_len,
                       s_len, inv_l, src);
  }
  return hipGetLastError();
}

// Varlen / paged: each sequence's last `last_n` complete kernels (all when
// last_n <= 0); the grid covers the most any sequence can have.
hipError_t launch_compress_k_varlen(const infv2_problem& p, const void* K,
                                    const int32_t* block_table, int max_blocks, int n_pages,
                                    const int32_t* seq_lens, void* Kc, int64_t kv_cap,
                                    int64_t c_cap, int l_len, int s_len, int last_n,
                                    hipStream_t stream) {
  const int n_max = p.n_kv < l_len ? 0 : (p.n_kv - l_len) / s_len + 1;
  const int n = last_n > 0 ? min(last_n, n_max) : n_max;
  if (n <= 0) return hipSuccess;
  const int per_blk = 256 / p.d;
  dim3 grid((n + per_blk - 1) / per_blk, p.h_kv, p.batch);
  dim3 block(per_blk * p.d);
  const double inv_l = 1.0 / (double)l_len;
  const CompressSrc src = {seq_lens, block_table, max_blocks, n_pages, p.B, p.n_q, p.n_kv, last_n};
  if (p.dtype == INFV2_BF16) {
    hipLaunchKernelGGL(compress_k_kernel<uint16_t>, grid, block, 0, stream,
                       (const uint16_t*)K, (uint16_t*)Kc, 0, 0, p.h_kv, p.d, kv_cap, c_cap,
                       l_len, s_len, inv_l, src);
  } else {
    hipLaunchKernelGGL(compress_k_kernel<float>, grid, block, 0, stream, (const float*)K,
                       (float*)Kc, 0, 0, p.h_kv, p.d, kv_cap, c_cap, l_len, s_len, inv_l, src);
  }
  return hipGetLastError();
}

}  // namespace infv2
