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
//  * V^T fragments need 8 consecutive keys of one feature: prefill reads them
//    from a transposed copy of V made once per call (vt_transpose_kernel);
//    decode stages each selected block through LDS.
//  * decode splits the selected blocks over workgroups (one block each) and
//    merges the partial (max, sum, O) afterwards.
// A generic fp64 kernel serves fp32 I/O and other shapes.
#include "common.hpp"

namespace infv2 {

constexpr int AT_D = 128;
constexpr int AT_G = 16;
constexpr int AT_B = 64;

// ---------------------------------------------------------------------------
// V [b][kv_cap][h_kv][d] -> VT [b][h_kv][d][n_pad]  (bf16), zero beyond n_kv.
// grid: x = 64-token tiles, y = h_kv, z = batch.  256 threads.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) vt_transpose_kernel(const uint16_t* __restrict__ V,
                                                           uint16_t* __restrict__ VT, int n_kv,
                                                           int n_pad, int h_kv, int64_t kv_cap) {
  __shared__ uint16_t tile[64][AT_D + 8];
  const int tt = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  // load 64 rows x 128 d: 1024 16-byte pieces, 4 per thread
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int u = tid + 256 * i;
    const int r = u >> 4, c8 = (u & 15) * 8;
    const int tok = tt * 64 + r;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (tok < n_kv) v = *(const u32x4*)(V + (((size_t)b * kv_cap + tok) * h_kv + g) * AT_D + c8);
    const uint16_t* e = (const uint16_t*)&v;
#pragma unroll
    for (int q = 0; q < 8; ++q) tile[r][c8 + q] = e[q];
  }
  __syncthreads();
  // write 128 d-rows x 64 tokens: thread -> (d, 32 tokens) as 4 x 16 B
  const int d = tid >> 1, half = tid & 1;
  uint16_t* dst = VT + (((size_t)b * h_kv + g) * AT_D + d) * n_pad + tt * 64 + half * 32;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = half * 32 + q * 8 + 2 * e;
      w[e] = (uint32_t)tile[r][d] | ((uint32_t)tile[r + 1][d] << 16);
    }
    *(u32x4*)(dst + q * 8) = u32x4{w[0], w[1], w[2], w[3]};
  }
}

// Key held by row r (0..15) of score tile t (0..3) of a 64-key block: the
// permutation makes a lane's 8 P^T elements of k-step ks the 8 consecutive
// keys 32*ks + 8*(lane>>4) .. +7.
__device__ __forceinline__ int tile_key(int t, int r) {
  return 32 * (t >> 1) + 8 * (r >> 2) + 4 * (t & 1) + (r & 3);
}

struct AttnArgs {
  const uint16_t* Q;
  const uint16_t* K;
  const uint16_t* VT;     // prefill: transposed V
  const uint16_t* V;      // decode: natural V
  const int32_t* idx;     // nullptr -> dense
  const int32_t* n_sel;
  uint16_t* O;
  float* lse;
  float* part_o;          // decode partials
  float2* part_ml;
  int n_q, q_pos0, n_kv, n_pad, h_kv, budget;
  int64_t kv_cap;
  float c;                // scale * log2(e)
};

// One block of 64 keys for one token's 16 heads: scores, online softmax, PV.
// kfrag(t, ks) returns the K fragment, vfrag(mt, ks) the V^T fragment.
template <typename KF, typename VF>
__device__ __forceinline__ void attn_block(const bf16x8 (&qf)[4], f32x4 (&o)[8], float& m_run,
                                           float& l_run, int kv0, int p, float c, int lane,
                                           KF kfrag, VF vfrag) {
  f32x4 s[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    s[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) s[t] = mfma16(kfrag(t, ks), qf[ks], s[t]);
  }
  const int grp = lane >> 4;
  float mx = kNegInf;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = kv0 + 32 * (t >> 1) + 8 * grp + 4 * (t & 1) + i;
      float x = s[t][i] * c;
      if (key > p) x = kNegInf;
      s[t][i] = x;
      mx = fmaxf(mx, x);
    }
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
  // P^T as bf16 B operands (k-step ks covers keys 32ks + 8*grp .. +7)
  bf16x8 pf[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = 2 * ks + (e >> 1);
      const int i0 = 2 * (e & 1);
      const float p0 = fast_exp2(s[t][i0] - m_new);
      const float p1 = fast_exp2(s[t][i0 + 1] - m_new);
      l_run += p0 + p1;                      // fp32 sum: exact-to-fp32 LSE
      w[e] = f32_to_bf16_bits(p0) | (f32_to_bf16_bits(p1) << 16);
    }
    pf[ks] = as_bf16x8(u32x4{w[0], w[1], w[2], w[3]});
  }
#pragma unroll
  for (int mt = 0; mt < 8; ++mt)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) o[mt] = mfma16(vfrag(mt, ks), pf[ks], o[mt]);
}

__device__ __forceinline__ void load_qfrag(const AttnArgs& a, int b, int t, int g, int lane,
                                           bf16x8 (&qf)[4]) {
  const int hq = a.h_kv * AT_G;
  const uint16_t* q = a.Q + (((size_t)b * a.n_q + t) * hq + g * AT_G + (lane & 15)) * AT_D;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) qf[ks] = as_bf16x8(*(const u32x4*)(q + 32 * ks + 8 * (lane >> 4)));
}

// grid: x = ceil(n_q/4) token quads, y = h_kv, z = batch; 4 waves = 4 tokens.
template <bool SPARSE>
__global__ void __launch_bounds__(256) attn_prefill_kernel(AttnArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nquads = gridDim.x;
  const int quad = nquads - 1 - (int)blockIdx.x;      // late tokens (long rows) first
  const int t = quad * 4 + wave;
  const int g = blockIdx.y, b = blockIdx.z;
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
  const size_t kstride = (size_t)a.h_kv * AT_D;
  const uint16_t* kbase = a.K + (size_t)b * a.kv_cap * kstride + (size_t)g * AT_D;
  const uint16_t* vtbase = a.VT + ((size_t)b * a.h_kv + g) * AT_D * a.n_pad;
  const int grp = lane >> 4, r16 = lane & 15;
  for (int bi = 0; bi < nblocks; ++bi) {
    const int blk = SPARSE ? sel[bi] : bi;
    if (blk < 0 || blk > b_p) continue;            // only causal blocks
    const int kv0 = blk * AT_B;
    auto kfrag = [&](int tt, int ks) -> bf16x8 {
      const int key = kv0 + tile_key(tt, r16);
      u32x4 v = {0u, 0u, 0u, 0u};
      if (key < a.n_kv) v = *(const u32x4*)(kbase + (size_t)key * kstride + 32 * ks + 8 * grp);
      return as_bf16x8(v);
    };
    auto vfrag = [&](int mt, int ks) -> bf16x8 {
      const int d = 16 * mt + r16;
      return as_bf16x8(*(const u32x4*)(vtbase + (size_t)d * a.n_pad + kv0 + 32 * ks + 8 * grp));
    };
    attn_block(qf, o, m_run, l_run, kv0, p, a.c, lane, kfrag, vfrag);
  }
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  const float inv = 1.0f / l_run;
  const int hq = a.h_kv * AT_G;
  uint16_t* orow = a.O + (((size_t)b * a.n_q + t) * hq + g * AT_G + r16) * AT_D;
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) {
    const uint32_t w0 = f32_to_bf16_bits(o[mt][0] * inv) | (f32_to_bf16_bits(o[mt][1] * inv) << 16);
    const uint32_t w1 = f32_to_bf16_bits(o[mt][2] * inv) | (f32_to_bf16_bits(o[mt][3] * inv) << 16);
    *(uint2*)(orow + 16 * mt + 4 * grp) = make_uint2(w0, w1);
  }
  if (a.lse && grp == 0)
    a.lse[((size_t)b * hq + g * AT_G + r16) * a.n_q + t] = (m_run + fast_log2(l_run)) * kLn2;
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

// V^T of one 64-key block in LDS: row d holds the 64 keys of feature d as eight
// 16-byte slots; slot (key>>3) is stored at (key>>3) ^ (d & 7) so that both the
// transposing writes and the fragment reads are free of bank conflicts.
__device__ __forceinline__ int vt_slot(int d, int key8) { return key8 ^ (d & 7); }

__global__ void __launch_bounds__(64) attn_split_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t vt[AT_D][AT_B];
  const int lane = threadIdx.x;
  const int slot = blockIdx.x, g = blockIdx.y, bt = blockIdx.z;
  const int b = bt / a.n_q, t = bt % a.n_q;
  const size_t row = ((size_t)b * a.h_kv + g) * a.n_q + t;
  const size_t prow = row * a.budget + slot;
  const int nsel = a.n_sel[row];
  if (slot >= nsel) return;
  const int p = a.q_pos0 + t;
  const int blk = a.idx[row * a.budget + slot];
  if (blk < 0 || blk > p / AT_B) {                  // only causal blocks
    if (lane < AT_G) a.part_ml[prow * AT_G + lane] = make_float2(kNegInf, 0.f);
    return;
  }
  const int kv0 = blk * AT_B;
  const size_t kstride = (size_t)a.h_kv * AT_D;
  const uint16_t* kbase = a.K + (size_t)b * a.kv_cap * kstride + (size_t)g * AT_D;
  const uint16_t* vbase = a.V + (size_t)b * a.kv_cap * kstride + (size_t)g * AT_D;
  // stage V^T: lane handles (key group kg of 8 keys, feature chunk c of 8)
  // for c = lane>>3 and c+8; 8 row loads, an 8x8 transpose, 8 slot writes.
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int kg = lane & 7, c = (lane >> 3) + 8 * half;
    u32x4 in[8], out[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int key = kv0 + 8 * kg + r;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (key < a.n_kv) v = *(const u32x4*)(vbase + (size_t)key * kstride + 8 * c);
      in[r] = v;
    }
    transpose8x8_bf16(in, out);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int d = 8 * c + q;
      *(u32x4*)(&vt[d][8 * vt_slot(d, kg)]) = out[q];
    }
  }
  __syncthreads();
  bf16x8 qf[4];
  load_qfrag(a, b, t, g, lane, qf);
  f32x4 o[8];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) o[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegInf, l_run = 0.f;
  const int grp = lane >> 4, r16 = lane & 15;
  auto kfrag = [&](int tt, int ks) -> bf16x8 {
    const int key = kv0 + tile_key(tt, r16);
    u32x4 v = {0u, 0u, 0u, 0u};
    if (key < a.n_kv) v = *(const u32x4*)(kbase + (size_t)key * kstride + 32 * ks + 8 * grp);
    return as_bf16x8(v);
  };
  auto vfrag = [&](int mt, int ks) -> bf16x8 {
    const int d = 16 * mt + r16;
    return as_bf16x8(*(const u32x4*)(&vt[d][8 * vt_slot(d, 4 * ks + grp)]));
  };
  attn_block(qf, o, m_run, l_run, kv0, p, a.c, lane, kfrag, vfrag);
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  // partial O^T (unnormalised) and (max, sum) per head
  float* po = a.part_o + prow * AT_G * AT_D;
#pragma unroll
  for (int mt = 0; mt < 8; ++mt)
    *(f32x4*)(po + (size_t)r16 * AT_D + 16 * mt + 4 * grp) = o[mt];
  if (grp == 0) a.part_ml[prow * AT_G + r16] = make_float2(m_run, l_run);
}

// grid: x = h_kv, y = batch*n_q; 256 threads: head = tid/16, 8 features each.
__global__ void __launch_bounds__(256) attn_merge_kernel(AttnArgs a) {
  const int g = blockIdx.x, bt = blockIdx.y;
  const int b = bt / a.n_q, t = bt % a.n_q;
  const size_t row = ((size_t)b * a.h_kv + g) * a.n_q + t;
  const int nsel = a.n_sel[row];
  const int h = threadIdx.x >> 4, d0 = (threadIdx.x & 15) * 8;
  float m = kNegInf;
  for (int s = 0; s < nsel; ++s) m = fmaxf(m, a.part_ml[(row * a.budget + s) * AT_G + h].x);
  float l = 0.f, acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < nsel; ++s) {
    const float2 ml = a.part_ml[(row * a.budget + s) * AT_G + h];
    if (ml.x == kNegInf) continue;
    const float w = fast_exp2(ml.x - m);
    l += ml.y * w;
    const float* po = a.part_o + ((row * a.budget + s) * AT_G + h) * AT_D + d0;
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] += po[q] * w;
  }
  const float inv = 1.0f / l;
  const int hq = a.h_kv * AT_G;
  uint16_t* orow = a.O + (((size_t)b * a.n_q + t) * hq + g * AT_G + h) * AT_D + d0;
  uint32_t w[4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
    w[q] = f32_to_bf16_bits(acc[2 * q] * inv) | (f32_to_bf16_bits(acc[2 * q + 1] * inv) << 16);
  *(u32x4*)orow = u32x4{w[0], w[1], w[2], w[3]};
  if (a.lse && (threadIdx.x & 15) == 0)
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
  const size_t n_pad = ((size_t)p.n_kv + 63) & ~(size_t)63;
  return (size_t)p.batch * p.h_kv * AT_D * n_pad * sizeof(uint16_t);
}

static AttnArgs fast_args(const infv2_problem& p, const void* Q, const void* K, const void* V,
                          const int32_t* idx, const int32_t* n_sel, void* O, float* lse,
                          int budget, int64_t kv_cap, float scale) {
  AttnArgs a;
  a.Q = (const uint16_t*)Q;
  a.K = (const uint16_t*)K;
  a.V = (const uint16_t*)V;
  a.VT = nullptr;
  a.idx = idx;
  a.n_sel = n_sel;
  a.O = (uint16_t*)O;
  a.lse = lse;
  a.part_o = nullptr;
  a.part_ml = nullptr;
  a.n_q = p.n_q;
  a.q_pos0 = p.q_pos0;
  a.n_kv = p.n_kv;
  a.n_pad = (p.n_kv + 63) & ~63;
  a.h_kv = p.h_kv;
  a.budget = budget;
  a.kv_cap = kv_cap;
  a.c = scale * kLog2e;
  return a;
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
      hipLaunchKernelGGL(attn_merge_kernel, dim3(p.h_kv, p.batch * p.n_q), dim3(256), 0, stream,
                         a);
      return hipGetLastError();
    }
    a.VT = (uint16_t*)ws;
    hipLaunchKernelGGL(vt_transpose_kernel, dim3(a.n_pad / 64, p.h_kv, p.batch), dim3(256), 0,
                       stream, (const uint16_t*)V, (uint16_t*)ws, p.n_kv, a.n_pad, p.h_kv, kv_cap);
    dim3 grid((p.n_q + 3) / 4, p.h_kv, p.batch);
    if (sparse)
      hipLaunchKernelGGL(attn_prefill_kernel<true>, grid, dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL(attn_prefill_kernel<false>, grid, dim3(256), 0, stream, a);
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
