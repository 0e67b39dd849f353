// Device-side helpers shared by the kernels of libinfv2 (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/infv2.h"

namespace infv2 {

// The compressed keys a selection call reads: K^C1 and, for the LSE
// approximation, K^C2 (else null), with their valid and allocated row counts.
struct KeySet {
  const void* Kc1;
  const void* Kc2;
  int n_c1, n_c2;
  int64_t c1_cap, c2_cap;
};

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

// bf16 <-> fp32 by bit manipulation (bf16 is the top half of an fp32).
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}
// fp32 -> bf16 bits, round to nearest even (inputs here are finite or inf).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Two fp32 values to packed bf16 (round to nearest even) with the hardware
// conversion (v_cvt_pk_bf16_f32 on gfx950); lo lands in the low half.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// 2^x on the transcendental unit (v_exp_f32).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Wave-level reductions (wave64).
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) {
  return __builtin_bit_cast(bf16x8, v);
}

// ---- cross-lane moves by the data-parallel primitives and permlane swaps.
// Every cross-lane read must run with all lanes active (a read from an
// inactive lane yields 0).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, CTRL, 0xF, 0xF, true);
}

// value of lane (lane ^ S), S = 1, 2, 4, 8, 16, 32
template <int S>
__device__ __forceinline__ uint32_t xor_lane(uint32_t x, int lane) {
  if constexpr (S == 1) {
    return dpp_u<0xB1>(x);                            // quad_perm [1,0,3,2]
  } else if constexpr (S == 2) {
    return dpp_u<0x4E>(x);                            // quad_perm [2,3,0,1]
  } else if constexpr (S == 4) {
    const uint32_t up = dpp_u<0x104>(x);              // row_shl:4  (lane + 4)
    const uint32_t dn = dpp_u<0x114>(x);              // row_shr:4  (lane - 4)
    return (lane & 4) ? dn : up;
  } else if constexpr (S == 8) {
    return dpp_u<0x128>(x);                           // row_ror:8 == lane ^ 8 within a row
  } else if constexpr (S == 16) {
    const auto sw = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    return (lane & 16) ? sw[0] : sw[1];
  } else {
    const auto sw = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return (lane & 32) ? sw[0] : sw[1];
  }
}

// Bitonic sort of one value per lane across the wave, descending (lane 0
// holds the largest); T = uint32_t or uint64_t.
template <typename T, int SIZE, int S>
__device__ __forceinline__ T bitonic_step(T v, int lane) {
  T o;
  if constexpr (sizeof(T) == 8) {
    const uint32_t lo = xor_lane<S>((uint32_t)v, lane);
    const uint32_t hi = xor_lane<S>((uint32_t)(v >> 32), lane);
    o = ((uint64_t)hi << 32) | lo;
  } else {
    o = xor_lane<S>(v, lane);
  }
  const bool keep_max = ((lane & SIZE) == 0) == ((lane & S) == 0);
  return keep_max ? (v > o ? v : o) : (v < o ? v : o);
}
template <typename T>
__device__ __forceinline__ T wave_sort_desc(T v, int lane) {
  v = bitonic_step<T, 2, 1>(v, lane);
  v = bitonic_step<T, 4, 2>(v, lane);  v = bitonic_step<T, 4, 1>(v, lane);
  v = bitonic_step<T, 8, 4>(v, lane);  v = bitonic_step<T, 8, 2>(v, lane);
  v = bitonic_step<T, 8, 1>(v, lane);
  v = bitonic_step<T, 16, 8>(v, lane); v = bitonic_step<T, 16, 4>(v, lane);
  v = bitonic_step<T, 16, 2>(v, lane); v = bitonic_step<T, 16, 1>(v, lane);
  v = bitonic_step<T, 32, 16>(v, lane); v = bitonic_step<T, 32, 8>(v, lane);
  v = bitonic_step<T, 32, 4>(v, lane);  v = bitonic_step<T, 32, 2>(v, lane);
  v = bitonic_step<T, 32, 1>(v, lane);
  v = bitonic_step<T, 64, 32>(v, lane); v = bitonic_step<T, 64, 16>(v, lane);
  v = bitonic_step<T, 64, 8>(v, lane);  v = bitonic_step<T, 64, 4>(v, lane);
  v = bitonic_step<T, 64, 2>(v, lane);  v = bitonic_step<T, 64, 1>(v, lane);
  return v;
}

// sum over the wave, in every lane: quads, rows (two rotations), then the
// row pairs and halves by permlane swaps
__device__ __forceinline__ int wave_sum_i(int v) {
  v += (int)dpp_u<0xB1>((uint32_t)v);                 // quad_perm [1,0,3,2]
  v += (int)dpp_u<0x4E>((uint32_t)v);                 // quad_perm [2,3,0,1]
  v += (int)dpp_u<0x124>((uint32_t)v);                // row_ror:4
  v += (int)dpp_u<0x128>((uint32_t)v);                // row_ror:8
  const auto s16 = __builtin_amdgcn_permlane16_swap((uint32_t)v, (uint32_t)v, false, false);
  v = (int)(s16[0] + s16[1]);
  const auto s32 = __builtin_amdgcn_permlane32_swap((uint32_t)v, (uint32_t)v, false, false);
  return (int)(s32[0] + s32[1]);
}

// Varlen batches: sequence b's cache length, clamped to [n_q, n_kv] so that a
// bad entry can never move a read past the buffers sized for n_kv.
__device__ __forceinline__ int seq_len_of(const int32_t* seq_lens, int b, int n_q, int n_kv) {
  return min(max(seq_lens[b], n_q), n_kv);
}

// order-preserving bits of a float (larger float -> larger unsigned)
__device__ __forceinline__ uint32_t ordered_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

}  // namespace infv2
