// Block selection I(p) = I_init u I_local(p) u top-k(p).
//
// papernotes.org InfLLM-V2 note, 方法详解 > 关键设计 2 (the union, top-k over the
// remaining blocks by S^cmp); OpenBMB blog "技术Blog-4 | 新一代InfLLM：可训练的稀疏
// 注意力机制", 动态上下文块选择 (initial and local blocks always attended) and
// Top-K块共享 (one selection per (token, group)).
//
// One wavefront per (token, group) row; the row's scores (up to 64 * NI
// blocks) are read once into registers as order-preserving 32-bit keys
// (candidates only; everything else is 0, below every candidate key).
// s* = the kk-th largest candidate key, counted with multiplicity:
//   1. the kk-th largest of the 64 lane maxima, K0, is a lower bound of s*;
//   2. the keys >= K0 (usually about kk of them) are gathered, one per lane,
//      and sorted across the wave; s* is the kk-th.  (If more than 64 keys
//      are >= K0 -- massive ties -- a bisection over the key range finds s*.)
// Selected: init/local blocks, candidates with key > s*, and, of the
// candidates with key == s*, the lowest-index ones up to kk in total -- ties
// go to the lower block index.  When the keys >= K0 were gathered (with their
// blocks, in block order), the list is written straight from them: init
// blocks, the selected gathered ones, local blocks.  Otherwise (bisection) the
// ascending list comes from a ballot/popcount compaction over every block.
// The sorts use lane moves of the data-parallel primitives and the permlane
// swaps only (no LDS round trips); every cross-lane read runs with all lanes
// active.
#include "common.hpp"

namespace infv2 {

struct TopkArgs {
  const float* S_cmp;
  int32_t* idx;
  int32_t* n_sel;
  int n_q, q_pos0, n_blk, B, k, N_init, N_local, budget;
  int rows;
};

// NI > 0: the row (nb <= 64*NI blocks) is held in NI registers per lane;
// NI == 0: any length, keys re-read from memory.
template <int NI>
__global__ void __launch_bounds__(256) topk_kernel(TopkArgs a) {
  __shared__ uint32_t gather_all[4][64];
  __shared__ int gblk_all[4][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row = blockIdx.x * 4 + wave;
  if (row >= a.rows) return;                 // whole wave leaves together
  uint32_t* gather = gather_all[wave];
  int* gblk = gblk_all[wave];
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
  const int niter = (nb + 63) >> 6;
  constexpr int NC = NI > 0 ? NI : 1;
  uint32_t kr[NC];
  auto key_of = [&](int blk, float v) -> uint32_t {
    return (blk >= init_hi && blk < loc_lo) ? ordered_bits(v) : 0u;
  };
  if constexpr (NI > 0) {
    float sc[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) sc[i] = srow[min(lane + 64 * i, nb - 1)];
#pragma unroll
    for (int i = 0; i < NI; ++i) kr[i] = key_of(lane + 64 * i, sc[i]);
  }
  auto key_at = [&](int i) -> uint32_t {
    if constexpr (NI > 0) return kr[i];
    const int blk = lane + 64 * i;
    return blk < nb ? key_of(blk, srow[blk]) : 0u;
  };
  auto count_ge = [&](uint32_t thr) -> int {
    int c = 0;
    if constexpr (NI > 0) {
#pragma unroll
      for (int i = 0; i < NI; ++i) c += kr[i] >= thr ? 1 : 0;
    } else {
      for (int i = 0; i < niter; ++i) c += key_at(i) >= thr ? 1 : 0;
    }
    return wave_sum_i(c);
  };
  // largest X with count(key >= X) >= kk, from a lower bound that satisfies it
  auto bisect = [&](uint32_t lo) -> uint32_t {
    uint32_t hi = 0xFFFFFFFFu;
    while (lo < hi) {
      const uint32_t mid = lo + ((hi - lo) >> 1) + 1;
      if (count_ge(mid) >= kk) lo = mid; else hi = mid - 1;
    }
    return lo;
  };

  uint32_t sstar = 0u;       // the kk-th largest candidate key
  const bool all = (kk == ncand);  // every candidate is selected
  int gathered = -1;         // >= 0: every key >= s* is in gather/gblk (that many)
  if (!all && kk > 0) {
    if (kk > 64) {
      sstar = bisect(1u);    // every candidate key is >= 1
    } else {
      uint32_t lmax = 0u;
      if constexpr (NI > 0) {
#pragma unroll
        for (int i = 0; i < NI; ++i) lmax = max(lmax, kr[i]);
      } else {
        for (int i = 0; i < niter; ++i) lmax = max(lmax, key_at(i));
      }
      const uint32_t sorted = wave_sort_desc<uint32_t>(lmax, lane);
      const uint32_t k0 = (uint32_t)__builtin_amdgcn_readlane((int)sorted, kk - 1);
      int cnt = 0;
      if constexpr (NI > 0) {
#pragma unroll
        for (int i = 0; i < NI; ++i) cnt += kr[i] >= k0 ? 1 : 0;
      } else {
        for (int i = 0; i < niter; ++i) cnt += key_at(i) >= k0 ? 1 : 0;
      }
      const int total = wave_sum_i(cnt);
      if (total <= 64) {
        // gather the keys >= k0, one per lane: positions by ballot and
        // count of set bits below this lane
        gather[lane] = 0u;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // (with their blocks: gathered in block order, so gblk ascends)
        int base = 0;
        auto put = [&](uint32_t kv, int blk) {
          const bool hit = kv >= k0;
          const uint64_t bal = __ballot(hit);
          if (hit) {
            const int at = base + (int)__popcll(bal & ((1ull << lane) - 1ull));
            gather[at] = kv;
            gblk[at] = blk;
          }
          base += (int)__popcll(bal);
        };
        if constexpr (NI > 0) {
#pragma unroll
          for (int i = 0; i < NI; ++i) put(kr[i], lane + 64 * i);
        } else {
          for (int i = 0; i < niter; ++i) put(key_at(i), lane + 64 * i);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const uint32_t s2 = wave_sort_desc<uint32_t>(gather[lane], lane);
        sstar = (uint32_t)__builtin_amdgcn_readlane((int)s2, kk - 1);
        gathered = total;
      } else {
        sstar = bisect(k0);                   // count(>= k0) >= kk holds
      }
    }
  }
  const uint64_t below = (1ull << lane) - 1ull;
  if (all || kk == 0 || gathered >= 0) {
    // the list is init blocks, the selected candidates (ascending), local
    // blocks: written directly, without a pass over every block.  With every
    // candidate selected (also when there is none: the local window then
    // reaches the init blocks) it is every block 0 .. b_p; otherwise
    // init_hi < loc_lo.
    const int n_sel = all ? nb : init_hi + kk + (nb - loc_lo);
    for (int j = lane; j < (all ? nb : init_hi); j += 64) out[j] = j;
    if (!all && kk > 0) {
      // of the gathered keys (block order): those > s*, and of those == s*
      // the lowest-index ones up to kk in total
      const uint32_t gk = lane < gathered ? gather[lane] : 0u;
      const bool gt = lane < gathered && gk > sstar;
      const bool eq = lane < gathered && gk == sstar;
      const int eq_take = kk - (int)__popcll(__ballot(gt));
      const bool sel = gt || (eq && (int)__popcll(__ballot(eq) & below) < eq_take);
      const int pos = init_hi + (int)__popcll(__ballot(sel) & below);
      if (sel) out[pos] = gblk[lane];
    }
    if (!all)
      for (int j = lane; j < nb - loc_lo; j += 64) out[init_hi + kk + j] = loc_lo + j;
    for (int i = n_sel + lane; i < a.budget; i += 64) out[i] = -1;
    if (lane == 0) a.n_sel[row] = n_sel;
    return;
  }
  // how many candidates equal to s* are taken (the lowest-index ones)
  int eq_left = 0;
  if (!all && kk > 0) {
    int c = 0;
    if constexpr (NI > 0) {
#pragma unroll
      for (int i = 0; i < NI; ++i) c += kr[i] > sstar ? 1 : 0;
    } else {
      for (int i = 0; i < niter; ++i) c += key_at(i) > sstar ? 1 : 0;
    }
    eq_left = kk - wave_sum_i(c);
  }
  // ascending compaction of the selected blocks (the bisection cases)
  int written = 0;
  auto emit = [&](int i) {
    const int blk = lane + 64 * i;
    const uint32_t kv = key_at(i);
    const bool cand = blk < nb && blk >= init_hi && blk < loc_lo;
    const bool fixed = blk < nb && !cand;
    const bool eq = cand && !all && kv == sstar;
    const uint64_t eq_ballot = __ballot(eq);
    const int eq_rank = (int)__popcll(eq_ballot & below);
    const bool sel = fixed || (cand && kk > 0 && (all || kv > sstar || (eq && eq_rank < eq_left)));
    eq_left -= (int)__popcll(eq_ballot);
    const uint64_t ballot = __ballot(sel);
    const int pos = written + (int)__popcll(ballot & below);
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
