// merge.hpp -- log-sum-exp merge of two attention results over disjoint key
// sets of the same rows (the prefix part and the causal suffix part of a
// shared-prefix branch). Memory-bound: one wave per row, 16-byte accesses.
// Each row's lse pair is read by every lane before lane 0 writes the merged
// lse, so lse may be updated in place; o may be o1 or o2 (each element is read
// and written by the same lane).
#pragma once
#include "common.hpp"

namespace gqa {

template <typename T>
__device__ __forceinline__ void load8(const T* src, float* x);
template <>
__device__ __forceinline__ void load8<float>(const float* src, float* x) {
  const f32x4 a = *(const f32x4*)src, b = *(const f32x4*)(src + 4);
  x[0] = a[0]; x[1] = a[1]; x[2] = a[2]; x[3] = a[3];
  x[4] = b[0]; x[5] = b[1]; x[6] = b[2]; x[7] = b[3];
}
template <>
__device__ __forceinline__ void load8<__bf16>(const __bf16* src, float* x) {
  const u32x4 u = *(const u32x4*)src;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(u[i] << 16);
    x[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
  }
}
template <>
__device__ __forceinline__ void load8<_Float16>(const _Float16* src, float* x) {
  typedef __attribute__((ext_vector_type(8))) _Float16 h8;
  const h8 u = *(const h8*)src;
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = (float)u[i];
}
template <typename T>
__device__ __forceinline__ void store8(T* dst, const float* x);
template <>
__device__ __forceinline__ void store8<float>(float* dst, const float* x) {
  *(f32x4*)dst = f32x4{x[0], x[1], x[2], x[3]};
  *(f32x4*)(dst + 4) = f32x4{x[4], x[5], x[6], x[7]};
}
template <>
__device__ __forceinline__ void store8<__bf16>(__bf16* dst, const float* x) {
  u32x4 u;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    typedef __attribute__((ext_vector_type(2))) __bf16 b2;
    b2 r;
    r[0] = (__bf16)x[2 * i];
    r[1] = (__bf16)x[2 * i + 1];
    u[i] = __builtin_bit_cast(unsigned, r);
  }
  *(u32x4*)dst = u;
}
template <>
__device__ __forceinline__ void store8<_Float16>(_Float16* dst, const float* x) {
  typedef __attribute__((ext_vector_type(8))) _Float16 h8;
  h8 u;
#pragma unroll
  for (int i = 0; i < 8; ++i) u[i] = (_Float16)x[i];
  *(h8*)dst = u;
}

template <typename T>
__global__ __launch_bounds__(256) void merge_kernel(const T* o1, const float* lse1, const T* o2, const float* lse2,
                                                    T* o, float* lse, int64_t rows, int64_t D) {
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= rows) return;
  const float a = lse1[r], b = lse2[r];
  const float M = fmaxf(a, b);
  float w1 = 0.f, w2 = 0.f, inv = 0.f, out_lse = -INFINITY;
  if (M != -INFINITY) {
    w1 = expf(a - M);
    w2 = expf(b - M);
    inv = 1.f / (w1 + w2);
    out_lse = M + logf(w1 + w2);
  }
  for (int64_t d = (int64_t)lane * 8; d < D; d += 512) {
    float x[8], y[8], z[8];
    load8<T>(o1 + r * D + d, x);
    load8<T>(o2 + r * D + d, y);
#pragma unroll
    for (int i = 0; i < 8; ++i) z[i] = (w1 * x[i] + w2 * y[i]) * inv;
    store8<T>(o + r * D + d, z);
  }
  // every lane of the wave read lse1[r], lse2[r] above, in program order
  if (lane == 0) lse[r] = out_lse;
}

// Merge of the n_split partial results of a split-KV forward (fp32 O parts
// [n_split][rows][D], lse parts [n_split][rows]) into o (in T) and lse: the
// same log-sum-exp combination over n_split disjoint key ranges. One
// workgroup per row (D = 256): wave 0 forms the max and the sum of the
// weights; then 8 groups of 32 lanes each take every 8th split (lane c of a
// group holds d 8c .. 8c + 7), with the loads of several splits in flight,
// and the 8 group sums meet in LDS. With many splits and few rows (decoding)
// a wave per row walking the splits one after another would wait on every
// load in turn.
constexpr int kMergeGroups = 8;
template <typename T>
__global__ __launch_bounds__(256) void merge_splits_kernel(const float* o_part, const float* lse_part, int n_split,
                                                           T* o, float* lse, int64_t rows) {
  __shared__ float part[kMergeGroups][kD];
  __shared__ float s_max, s_inv, s_lse;
  const int64_t r = blockIdx.x;
  const int t = threadIdx.x, lane = t & 63;
  if (t < 64) {
    float m = -INFINITY;
    for (int s = lane; s < n_split; s += 64) m = fmaxf(m, lse_part[(int64_t)s * rows + r]);
    for (int x = 32; x >= 1; x >>= 1) m = fmaxf(m, __shfl_xor(m, x));
    float sum = 0.f;
    if (m != -INFINITY)
      for (int s = lane; s < n_split; s += 64) sum += expf(lse_part[(int64_t)s * rows + r] - m);
    for (int x = 32; x >= 1; x >>= 1) sum += __shfl_xor(sum, x);
    if (lane == 0) {
      s_max = m;
      s_inv = sum > 0.f ? 1.f / sum : 0.f;
      s_lse = (m == -INFINITY) ? -INFINITY : m + logf(sum);
    }
  }
  __syncthreads();
  const float M = s_max, inv = s_inv;
  const int sg = t >> 5, c = t & 31;
  float z[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (M != -INFINITY) {
#pragma unroll 4
    for (int s = sg; s < n_split; s += kMergeGroups) {
      const float w = expf(lse_part[(int64_t)s * rows + r] - M) * inv;
      float x[8];
      load8<float>(o_part + ((int64_t)s * rows + r) * kD + 8 * c, x);
#pragma unroll
      for (int i = 0; i < 8; ++i) z[i] = fmaf(w, x[i], z[i]);
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) part[sg][8 * c + i] = z[i];
  __syncthreads();
  if (t < 32) {
    float y[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float acc = 0.f;
#pragma unroll
      for (int g2 = 0; g2 < kMergeGroups; ++g2) acc += part[g2][8 * t + i];
      y[i] = acc;
    }
    store8<T>(o + r * kD + 8 * t, y);
  }
  if (t == 0) lse[r] = s_lse;
}

}  // namespace gqa
