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
// workgroup per row (D = 256): 8 groups of 32 lanes take every 8th split
// (lane c of a group holds d 8c .. 8c + 7) and keep a running state over
// their splits -- max M, weight sum W = sum exp(lse_s - M), weighted sum
// Z = sum exp(lse_s - M) o_s -- that moves to a new max by one rescale. The
// splits come in batches of 8 per group whose loads (lse and O) are all
// issued before any of them is used, so a batch costs one round trip to
// memory (indexes past the last split load split sg again and are masked).
// The 8 group states then meet in LDS, rescaled to the common max.
constexpr int kMergeGroups = 8;
constexpr int kMergeBatch = 8;
template <typename T>
__global__ __launch_bounds__(256) void merge_splits_kernel(const float* o_part, const float* lse_part, int n_split,
                                                           T* o, float* lse, int64_t rows) {
  __shared__ float part[kMergeGroups][kD];
  __shared__ float gmax[kMergeGroups], gsum[kMergeGroups];
  const int64_t r = blockIdx.x;
  const int t = threadIdx.x, sg = t >> 5, c = t & 31;
  float m = -INFINITY, w = 0.f;
  float z[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int s0 = sg; s0 < n_split; s0 += kMergeBatch * kMergeGroups) {
    float a[kMergeBatch];
    f32x4 x[kMergeBatch][2];
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j) {
      const int s = s0 + j * kMergeGroups;
      const int sl = s < n_split ? s : sg;
      a[j] = lse_part[(int64_t)sl * rows + r];
      const float* src = o_part + ((int64_t)sl * rows + r) * kD + 8 * c;
      x[j][0] = *(const f32x4*)src;
      x[j][1] = *(const f32x4*)(src + 4);
    }
    // one statement takes every loaded value: all 24 loads are issued before
    // the first wait (left to itself the compiler interleaves loads and waits)
    asm volatile("" : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(a[4]), "+v"(a[5]), "+v"(a[6]),
                 "+v"(a[7]), "+v"(x[0][0]), "+v"(x[0][1]), "+v"(x[1][0]), "+v"(x[1][1]), "+v"(x[2][0]),
                 "+v"(x[2][1]), "+v"(x[3][0]), "+v"(x[3][1]), "+v"(x[4][0]), "+v"(x[4][1]), "+v"(x[5][0]),
                 "+v"(x[5][1]), "+v"(x[6][0]), "+v"(x[6][1]), "+v"(x[7][0]), "+v"(x[7][1]));
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j) {
      // an empty split (lse -inf, O 0) adds nothing; while every split so far
      // was empty the state stays (-inf, 0, 0)
      const float aj = s0 + j * kMergeGroups < n_split ? a[j] : -INFINITY;
      const float mn = fmaxf(m, aj);
      const float sc = mn == -INFINITY ? 1.f : expf(m - mn);
      const float e = mn == -INFINITY ? 0.f : expf(aj - mn);
      w = fmaf(w, sc, e);
#pragma unroll
      for (int i = 0; i < 8; ++i) z[i] = fmaf(z[i], sc, e * x[j][i >> 2][i & 3]);
      m = mn;
    }
  }
  if (c == 0) {
    gmax[sg] = m;
    gsum[sg] = w;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) part[sg][8 * c + i] = z[i];
  __syncthreads();
  if (t < 32) {
    float M = -INFINITY;
#pragma unroll
    for (int g2 = 0; g2 < kMergeGroups; ++g2) M = fmaxf(M, gmax[g2]);
    float tot = 0.f, y[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int g2 = 0; g2 < kMergeGroups; ++g2) {
      const float sc = gmax[g2] == -INFINITY ? 0.f : expf(gmax[g2] - M);
      tot = fmaf(sc, gsum[g2], tot);
#pragma unroll
      for (int i = 0; i < 8; ++i) y[i] = fmaf(sc, part[g2][8 * t + i], y[i]);
    }
    const float inv = tot > 0.f ? 1.f / tot : 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] *= inv;
    store8<T>(o + r * kD + 8 * t, y);
    if (t == 0) lse[r] = tot > 0.f ? M + logf(tot) : -INFINITY;
  }
}

}  // namespace gqa
