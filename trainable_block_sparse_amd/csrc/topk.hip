// Block selection I(p) = I_init u I_local(p) u top-k(p).
//
// papernotes.org InfLLM-V2 note, 方法详解 > 关键设计 2 (the union, top-k over the
// remaining blocks by S^cmp); OpenBMB blog "技术Blog-4 | 新一代InfLLM：可训练的稀疏
// 注意力机制", 动态上下文块选择 (initial and local blocks always attended) and
// Top-K块共享 (one selection per (token, group)).
//
// One wavefront per (token, group) row.  Every candidate block gets a unique
// 64-bit key  (order-preserving bits of S^cmp) << 32 | ~blk,  so a larger key
// means a larger score and, at equal scores, a lower block index.  The k-th
// largest key K* is found in two steps:
//   1. each lane takes the maximum key of its blocks (blk = lane + 64 i); the
//      kk-th largest of the 64 lane maxima, K0, is a lower bound of K*
//      (kk lanes hold a key >= K0);
//   2. the keys >= K0 (usually about kk of them) are gathered, one per lane,
//      and sorted across the wave; K* is the kk-th.  If more than 64 keys
//      are >= K0 a bisection over the 64-bit key range finds K* instead.
// Rows of up to 2048 blocks are read once, in one burst, into registers.
// Membership is then  init/local, or key >= K*;  the ascending index list
// comes from a ballot/popcount compaction over the blocks in order.
#include "common.hpp"

namespace infv2 {

__device__ __forceinline__ uint32_t ordered_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  const uint32_t lo = __shfl_xor((uint32_t)v, m, 64);
  const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), m, 64);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t shfl_u64(uint64_t v, int src) {
  const uint32_t lo = __shfl((uint32_t)v, src, 64);
  const uint32_t hi = __shfl((uint32_t)(v >> 32), src, 64);
  return ((uint64_t)hi << 32) | lo;
}

// Bitonic sort across the 64 lanes, descending (lane 0 holds the largest).
__device__ __forceinline__ uint64_t wave_sort_desc(uint64_t v, int lane) {
#pragma unroll
  for (int size = 2; size <= 64; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      const uint64_t o = shfl_xor_u64(v, stride);
      const bool up = (lane & size) == 0;            // this run sorts descending
      const bool lower = (lane & stride) == 0;       // this lane keeps the larger
      const bool keep_max = (up == lower);
      v = keep_max ? (v > o ? v : o) : (v < o ? v : o);
    }
  }
  return v;
}

struct TopkArgs {
  const float* S_cmp;
  int32_t* idx;
  int32_t* n_sel;
  int n_q, q_pos0, n_blk, B, k, N_init, N_local, budget;
  int rows;
};

// NI > 0: the row (nb <= 64*NI blocks) is loaded once, in one burst, into
// NI registers per lane; NI == 0: any length, scores re-read from memory.
template <int NI>
__global__ void __launch_bounds__(256) topk_kernel(TopkArgs a) {
  __shared__ uint64_t gather_all[4][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row = blockIdx.x * 4 + wave;
  if (row >= a.rows) return;                 // whole wave leaves together
  uint64_t* gather = gather_all[wave];
  const int t = row % a.n_q;
  const int p = a.q_pos0 + t;
  const int b_p = p / a.B;
  const int nb = b_p + 1;
  const int init_hi = min(a.N_init, nb);                    // [0, init_hi)
  const int loc_lo = max(0, b_p - a.N_local + 1);           // [loc_lo, nb)
  const int ncand = max(0, loc_lo - init_hi);               // blocks in between
  const int kk = min(a.k, ncand);
  const float* srow = a.S_cmp + (size_t)row * a.n_blk;
  int32_t* out = a.idx + (size_t)row * a.budget;
  constexpr int NC = NI > 0 ? NI : 1;
  float sc[NC];
  if constexpr (NI > 0) {
#pragma unroll
    for (int i = 0; i < NI; ++i) sc[i] = srow[min(lane + 64 * i, nb - 1)];
  }
  const int niter = (nb + 63) >> 6;
  auto key_at = [&](int i) -> uint64_t {     // key of block lane + 64*i
    const int blk = lane + 64 * i;
    if (blk >= nb || blk < init_hi || blk >= loc_lo) return 0ull;   // not a candidate
    float v;
    if constexpr (NI > 0) v = sc[i]; else v = srow[blk];
    return ((uint64_t)ordered_bits(v) << 32) | (uint64_t)(~(uint32_t)blk);
  };
  auto count_ge = [&](uint64_t thr) -> int {
    int c = 0;
    if constexpr (NI > 0) {
#pragma unroll
      for (int i = 0; i < NI; ++i) c += key_at(i) >= thr ? 1 : 0;
    } else {
      for (int i = 0; i < niter; ++i) c += key_at(i) >= thr ? 1 : 0;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o, 64);
    return c;
  };
  // largest X with count(key >= X) >= kk, starting from a known lower bound
  auto bisect = [&](uint64_t lo) -> uint64_t {
    uint64_t hi = ~0ull;
    while (lo < hi) {
      const uint64_t mid = lo + ((hi - lo) >> 1) + 1;
      if (count_ge(mid) >= kk) lo = mid; else hi = mid - 1;
    }
    return lo;
  };

  uint64_t kstar = 0ull;     // keys >= kstar are selected
  const bool all = (kk == ncand);  // every candidate is selected
  if (all || kk == 0) {
    // nothing to rank
  } else if (kk > 64) {
    kstar = bisect(1ull);    // every candidate key is >= 1, non-candidates are 0
  } else {
    uint64_t lmax = 0ull;
    if constexpr (NI > 0) {
#pragma unroll
      for (int i = 0; i < NI; ++i) { const uint64_t kv = key_at(i); lmax = kv > lmax ? kv : lmax; }
    } else {
      for (int i = 0; i < niter; ++i) { const uint64_t kv = key_at(i); lmax = kv > lmax ? kv : lmax; }
    }
    const uint64_t sorted = wave_sort_desc(lmax, lane);
    const uint64_t k0 = shfl_u64(sorted, kk - 1);
    // count and gather the keys >= k0
    int cnt = 0;
    if constexpr (NI > 0) {
#pragma unroll
      for (int i = 0; i < NI; ++i) cnt += key_at(i) >= k0 ? 1 : 0;
    } else {
      for (int i = 0; i < niter; ++i) cnt += key_at(i) >= k0 ? 1 : 0;
    }
    int total = cnt;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) total += __shfl_xor(total, o, 64);
    if (total <= 64) {
      int pre = cnt;                          // exclusive prefix of cnt over lanes
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(pre, o, 64);
        if (lane >= o) pre += v;
      }
      pre -= cnt;
      gather[lane] = 0ull;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      if constexpr (NI > 0) {
#pragma unroll
        for (int i = 0; i < NI; ++i) { const uint64_t kv = key_at(i); if (kv >= k0) gather[pre++] = kv; }
      } else {
        for (int i = 0; i < niter; ++i) { const uint64_t kv = key_at(i); if (kv >= k0) gather[pre++] = kv; }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const uint64_t s2 = wave_sort_desc(gather[lane], lane);
      kstar = shfl_u64(s2, kk - 1);
    } else {
      kstar = bisect(k0);                     // count(>= k0) >= kk holds
    }
  }
  // ascending compaction of the selected blocks
  int written = 0;
  auto emit = [&](int i) {
    const int blk = lane + 64 * i;
    bool sel = false;
    if (blk < nb) {
      if (blk < init_hi || blk >= loc_lo) sel = true;
      else sel = all || (kk > 0 && key_at(i) >= kstar);
    }
    const uint64_t ballot = __ballot(sel);
    const int pos = written + (int)__popcll(ballot & ((1ull << lane) - 1ull));
    if (sel) out[pos] = blk;
    written += (int)__popcll(ballot);
  };
  if constexpr (NI > 0) {
#pragma unroll
    for (int i = 0; i < NI; ++i) if (i < niter) emit(i);
  } else {
    for (int i = 0; i < niter; ++i) emit(i);
  }
  for (int i = written + lane; i < a.budget; i += 64) out[i] = -1;
  if (lane == 0) a.n_sel[row] = written;
}

hipError_t launch_topk(const infv2_problem& p, const float* S_cmp, int32_t* idx, int32_t* n_sel,
                       int n_blk, int budget, hipStream_t stream) {
  TopkArgs a;
  a.S_cmp = S_cmp;
  a.idx = idx;
  a.n_sel = n_sel;
  a.n_q = p.n_q;
  a.q_pos0 = p.q_pos0;
  a.n_blk = n_blk;
  a.B = p.B;
  a.k = p.k;
  a.N_init = p.N_init;
  a.N_local = p.N_local;
  a.budget = budget;
  a.rows = p.batch * p.h_kv * p.n_q;
  dim3 grid((a.rows + 3) / 4);
  if (n_blk <= 256)
    hipLaunchKernelGGL(topk_kernel<4>, grid, dim3(256), 0, stream, a);
  else if (n_blk <= 1024)
    hipLaunchKernelGGL(topk_kernel<16>, grid, dim3(256), 0, stream, a);
  else if (n_blk <= 2048)
    hipLaunchKernelGGL(topk_kernel<32>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(topk_kernel<0>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace infv2
