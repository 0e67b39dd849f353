// The exact mean of one kernel's keys (K^C1: l_C1 keys at stride s_C1; K^C2:
// 4 l_C1 at 4 s_C1), shared by the compress kernels and the decode logits
// kernel that appends the step's kernel on the fly, so that both round
// identically.
//
// papernotes.org InfLLM-V2 note, 方法详解 > 关键设计 3 (the representation of a
// kernel is the mean of its keys); OpenBMB blog "技术Blog-4 | 新一代InfLLM：可训练的
// 稀疏注意力机制", 动态上下文块选择 > 语义核.
//
// The sum of the keys is carried as an fp64 pair (hi, lo) with TwoSum, keys
// added in order: exact unless the kernel's values span more than about 78
// binades (never for bf16 or fp32 data of one attention layer in practice);
// the pair is renormalised, scaled by 1/l (a power of two: exact) and rounded
// ONCE to the I/O format, to nearest even.
#pragma once

#include "common.hpp"

namespace infv2 {

// Round (hi + lo) to a binary format with P significant bits and fp32's
// exponent range, to nearest even; |lo| <= ulp(hi)/2 (a TwoSum pair).
template <int P>
__device__ __forceinline__ double round_pair(double hi, double lo) {
  if (hi == 0.0 || !__builtin_isfinite(hi)) return hi + lo;
  int e;
  (void)__builtin_frexp(hi, &e);             // hi = m * 2^e, 0.5 <= |m| < 1
  int qexp = e - P;
  if (qexp < -126 - P + 1) qexp = -126 - P + 1;   // subnormal quantum
  const double scaled = __builtin_ldexp(hi, -qexp);
  double r = __builtin_rint(scaled);         // ties to even
  const double delta = scaled - r;           // exact
  if ((delta == 0.5 || delta == -0.5) && lo != 0.0) {
    // hi sits exactly on a midpoint: the sign of lo decides the direction.
    if ((lo > 0.0) == (delta > 0.0)) r += (delta > 0.0) ? 1.0 : -1.0;
  }
  return __builtin_ldexp(r, qexp);
}

// one key value into the running pair (TwoSum error accumulated in lo)
__device__ __forceinline__ void kmean_add(double& hi, double& lo, double x) {
  const double t = hi + x;
  const double bp = t - hi;
  lo += (hi - (t - bp)) + (x - bp);
  hi = t;
}

// the pair renormalised (|lo| <= ulp(hi)/2) and scaled by inv_l
__device__ __forceinline__ void kmean_finish(double hi, double lo, double inv_l, double& rh,
                                             double& rl) {
  const double t = hi + lo;
  const double bp = t - hi;
  const double e = (hi - (t - bp)) + (lo - bp);
  rh = t * inv_l;
  rl = e * inv_l;
}

// the rounded mean as bf16 bits
__device__ __forceinline__ uint16_t kmean_bf16(double rh, double rl) {
  const float r = (float)round_pair<8>(rh, rl);      // exact: 8 bits fit fp32
  return (uint16_t)(__float_as_uint(r) >> 16);        // exact: low half is zero
}

// Features 2f, 2f+1 of kernel j of one sequence and group, as two bf16 in one
// word: keys j*s_len .. j*s_len + l_len - 1 of the rows at `col` (the
// sequence's first key row, offset to the group and to feature 2f),
// row_stride elements apart.  The loads of each 32 keys are all issued before
// the sums, which add the keys in order (the same operations as the compress
// kernel, -0 padding included).
__device__ __forceinline__ uint32_t kmean_pair_bf16(const uint16_t* col, size_t row_stride, int j,
                                                    int l_len, int s_len, double inv_l) {
  double h0 = 0.0, l0 = 0.0, h1 = 0.0, l1 = 0.0;
  const uint16_t* src = col + (size_t)j * s_len * row_stride;
  for (int u0 = 0; u0 < l_len; u0 += 32) {
    const int cnt = min(32, l_len - u0);
    uint32_t w[32];
#pragma unroll
    for (int u = 0; u < 32; ++u)
      w[u] = *(const uint32_t*)(src + (size_t)(u0 + min(u, cnt - 1)) * row_stride);
#pragma unroll
    for (int u = 0; u < 32; ++u) {
      const bool in = u < cnt;
      kmean_add(h0, l0, in ? (double)bf16_bits_to_f32(w[u] & 0xffffu) : -0.0);
      kmean_add(h1, l1, in ? (double)bf16_bits_to_f32(w[u] >> 16) : -0.0);
    }
  }
  double a0, b0, a1, b1;
  kmean_finish(h0, l0, inv_l, a0, b0);
  kmean_finish(h1, l1, inv_l, a1, b1);
  return (uint32_t)kmean_bf16(a0, b0) | ((uint32_t)kmean_bf16(a1, b1) << 16);
}

}  // namespace infv2
