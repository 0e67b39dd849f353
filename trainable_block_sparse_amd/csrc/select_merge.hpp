// Merge of a decode row's per-chunk candidate lists into its block set, by one
// wave (the workgroup is that one wave).
//
// The selection's pool stage leaves, for every chunk of 64 blocks, its kc best
// candidate blocks as sorted 64-bit keys: order-preserving score bits << 32 |
// ~block (unique; at equal scores the lower block ranks higher; 0 = none).
// The row's set is I(p) = init blocks (the first N_init) u local blocks (the
// last N_local up to the token's own block b_p) u the kk = min(k, #candidates)
// best candidates (OpenBMB blog, 动态上下文块选择 and 高效Top-K实现; papernotes
// note, 关键设计 2), listed in ascending block order.
//
// The kk best keys are found without sorting every key: the best r keys of
// each list (r = ceil(kk / lists)) are real keys, so their kk-th largest is a
// lower bound for the kk-th best key K*; the keys at or above that bound (a
// few more than kk as a rule) are gathered and sorted by the wave, and its
// first kk lanes are the selection.  With more than 64 keys at the bound
// (heavy ties), each such key is ranked against every key instead.  Selected:
// init, local, and every candidate key >= K* -- the same set as the
// 256-thread merge kernel of the selection.  Everything stays in registers
// but a 64-word gather buffer; the keys arrive in one memory round trip.
#pragma once

#include "common.hpp"

namespace infv2 {

// Where the selection's pool stage left the candidate lists: [rows][nch][kc].
struct CandLists {
  const uint64_t* cand;
  int nch, kc;
};

constexpr int SM_MAX_KEYS = 1024;    // lists x keys per list, per row

__device__ __forceinline__ uint64_t lane_u64(uint64_t v, int src) {
  const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, src);
  const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(v >> 32), src);
  return ((uint64_t)hi << 32) | lo;
}

// Position of the calling lane among the lanes set in m below it.
__device__ __forceinline__ int lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// A row's set, as list entries: entries [0, init_hi) are blocks 0 .. init_hi-1,
// entries [init_hi, init_hi + kk) the selected candidates in ascending order
// (lane i of mid holds the i-th), the rest the local blocks from loc_lo on
// (loc_lo >= init_hi).
struct RowSel {
  int init_hi, kk, loc_lo, n_sel;
  uint32_t mid;
};

__device__ __forceinline__ int row_sel_block(const RowSel& r, int s) {
  if (s < r.init_hi) return s;
  if (s < r.init_hi + r.kk) return (int)__builtin_amdgcn_readlane(r.mid, s - r.init_hi);
  return r.loc_lo + (s - r.init_hi - r.kk);
}

// The keys at or above `bound` among the row's nkeys keys (kv[m] holds key
// lane + 64 m), in list order, into pick[0 .. 64); returns how many there are.
__device__ __forceinline__ int pick_at_least(const uint64_t (&kv)[SM_MAX_KEYS / 64], int nkeys,
                                             uint64_t bound, int lane, uint64_t* pick) {
  int total = 0;
#pragma unroll
  for (int m = 0; m < SM_MAX_KEYS / 64; ++m) {
    if (64 * m >= nkeys) break;
    const bool take = 64 * m + lane < nkeys && kv[m] >= bound;
    const uint64_t bal = __ballot(take);
    const int pos = total + lanes_below(bal);
    if (take && pos < 64) pick[pos] = kv[m];
    total += __builtin_popcountll(bal);
  }
  return total;
}

// Merges the row's nch_all lists of kc keys at rlist into its set (64
// threads, one wave; pick: 64 words of LDS).  Requires nch_all * kc <=
// SM_MAX_KEYS and N_init + N_local + k <= 64.
__device__ __forceinline__ RowSel sel_merge_wave(const uint64_t* rlist, int nch_all, int kc, int k,
                                                 int N_init, int N_local, int b_p, int lane,
                                                 uint64_t* pick) {
  RowSel r;
  const int nb = b_p + 1;
  r.init_hi = min(N_init, nb);
  // local blocks from max(b_p - N_local + 1, init_hi): an early token's local
  // window may reach into the init blocks, which are listed once
  r.loc_lo = max(max(0, b_p - N_local + 1), r.init_hi);
  const int ncand = max(0, r.loc_lo - r.init_hi);
  r.kk = min(k, ncand);
  r.n_sel = r.init_hi + r.kk + (nb - r.loc_lo);
  r.mid = (uint32_t)(r.init_hi + lane);      // every candidate selected (kk == ncand)
  if (r.kk == 0 || r.kk == ncand) return r;
  // only the lists of chunks that hold candidates (blocks < loc_lo) count
  const int nch = min(nch_all, (r.loc_lo + 63) >> 6);
  const int nkeys = nch * kc;
  const int kk = r.kk;
  // every load in one round trip: the best rr keys of each list, and all keys
  const int rr = (kk + nch - 1) / nch;     // nch * rr <= 64 as kk <= 32, nch <= 64
  const uint64_t e = lane < nch * rr ? rlist[(lane / rr) * kc + lane % rr] : 0ull;
  uint64_t kv[SM_MAX_KEYS / 64];
#pragma unroll
  for (int m = 0; m < SM_MAX_KEYS / 64; ++m)
    kv[m] = 64 * m + lane < nkeys ? rlist[64 * m + lane] : 0ull;
  // a lower bound for the kk-th best key K*: the kk-th best of those heads
  const uint64_t hs = wave_sort_desc<uint64_t>(e, lane);
  uint64_t bound = lane_u64(hs, kk - 1);
  bound = bound > 1ull ? bound : 1ull;
  const int total = pick_at_least(kv, nkeys, bound, lane, pick);
  __syncthreads();
  uint64_t top;                              // lane i < kk: the i-th best key
  if (total <= 64) {
    top = wave_sort_desc<uint64_t>(lane < total ? pick[lane] : 0ull, lane);
  } else {
    // many keys at or above the bound (ties): rank each against every key
    // (keys are unique, so exactly one has kk - 1 keys above it), then take
    // the kk keys at or above it
    uint64_t found = 0ull;
#pragma unroll
    for (int m = 0; m < SM_MAX_KEYS / 64; ++m) {
      if (64 * m >= nkeys) break;
      if (64 * m + lane >= nkeys || kv[m] < bound) continue;
      int above = 0;
      for (int j = 0; j < nkeys; ++j) above += rlist[j] > kv[m] ? 1 : 0;
      if (above == kk - 1) found = kv[m];
    }
    const uint64_t fm = __ballot(found != 0ull);
    const uint64_t kstar = fm ? lane_u64(found, __builtin_ctzll(fm)) : 1ull;
    __syncthreads();
    pick_at_least(kv, nkeys, kstar, lane, pick);
    __syncthreads();
    top = lane < kk ? pick[lane] : 0ull;
  }
  // the kk selected candidates in ascending block order
  const uint32_t inv = lane < kk ? 0xffffffffu - ~(uint32_t)top : 0u;
  r.mid = 0xffffffffu - wave_sort_desc<uint32_t>(inv, lane);
  return r;
}

// The row's list: idx[0 .. n_sel) ascending, -1 after it up to budget (<= 64).
__device__ __forceinline__ void sel_write_list(const RowSel& r, int32_t* out, int budget, int lane) {
  const uint32_t m = __shfl(r.mid, min(max(lane - r.init_hi, 0), 63), 64);
  if (lane >= budget) return;
  int v = -1;
  if (lane < r.n_sel) {
    if (lane < r.init_hi) v = lane;
    else if (lane < r.init_hi + r.kk) v = (int)m;
    else v = r.loc_lo + (lane - r.init_hi - r.kk);
  }
  out[lane] = v;
}

}  // namespace infv2
