// Merge of split-key partial attention results.
//
// When a sequence's key range is split across workgroups, each part yields an
// output normalised over its own keys and the log-sum-exp of its scaled
// scores.  The full result is the log-sum-exp-weighted average of the parts:
//   lse = log sum_i exp(lse_i),   O = sum_i exp(lse_i - lse) O_i.
// Parts with lse_i = -inf (no keys) carry zero weight; if every part is empty
// the output is 0 and lse is -inf.
//
// One thread per (row, head, 4 dims): a wave covers 4 (row, head) pairs, so
// each part's load instruction reads 1 KiB of contiguous partials, and each
// thread keeps 16 parts' loads (16 bytes each) in flight at once.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernels.hpp"

namespace kvc {
namespace {

constexpr int D = kHeadDim;

typedef float floatx4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef __bf16 bf16x4 __attribute__((__vector_size__(4 * sizeof(__bf16))));
typedef _Float16 halfx4 __attribute__((__vector_size__(4 * sizeof(_Float16))));

template <typename T>
__device__ __forceinline__ void store_out(T* o, size_t i, floatx4 v);
template <>
__device__ __forceinline__ void store_out<uint16_t>(uint16_t* o, size_t i, floatx4 v) {
  *reinterpret_cast<bf16x4*>(o + i) = __builtin_convertvector(v, bf16x4);
}
template <>
__device__ __forceinline__ void store_out<float>(float* o, size_t i, floatx4 v) {
  *reinterpret_cast<floatx4*>(o + i) = v;
}

template <typename T>
__global__ __launch_bounds__(256) void attn_merge_kernel(int parts, int rows_heads, const float* __restrict__ po,
                                                         const float* __restrict__ plse, T* __restrict__ o,
                                                         float* __restrict__ lse) {
  const int rh = blockIdx.x * 16 + (threadIdx.x >> 4);
  const int d4 = (threadIdx.x & 15) * 4;
  if (rh >= rows_heads) return;
  // Parts are consumed in batches of 16 whose loads are all issued together;
  // the running maximum m keeps the weights finite across batches.
  constexpr int B = 16;
  float m = -INFINITY, z = 0.f;
  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int i0 = 0; i0 < parts; i0 += B) {
    float li[B];
    floatx4 oi[B];
#pragma unroll
    for (int j = 0; j < B; ++j) {
      const int i = i0 + j;
      const bool ok = i < parts;
      li[j] = ok ? plse[static_cast<size_t>(i) * rows_heads + rh] : -INFINITY;
      oi[j] = ok ? *reinterpret_cast<const floatx4*>(po + (static_cast<size_t>(i) * rows_heads + rh) * D + d4)
                 : floatx4{0.f, 0.f, 0.f, 0.f};
    }
    float mb = li[0];
#pragma unroll
    for (int j = 1; j < B; ++j) mb = fmaxf(mb, li[j]);
    if (mb == -INFINITY) continue;
    if (mb > m) {
      const float c = m == -INFINITY ? 0.f : __expf(m - mb);
      z *= c;
      acc *= c;
      m = mb;
    }
#pragma unroll
    for (int j = 0; j < B; ++j) {
      const float w = li[j] == -INFINITY ? 0.f : __expf(li[j] - m);
      z += w;
#pragma unroll
      for (int k = 0; k < 4; ++k) acc[k] = __builtin_fmaf(w, oi[j][k], acc[k]);
    }
  }
  floatx4 out;
#pragma unroll
  for (int k = 0; k < 4; ++k) out[k] = z > 0.f ? acc[k] / z : 0.f;
  store_out<T>(o, static_cast<size_t>(rh) * D + d4, out);
  if (lse && d4 == 0) lse[rh] = z > 0.f ? m + __logf(z) : -INFINITY;
}

// The same merge over partials in the fp16 form of the bf16 and FP8 attention
// kernels: part i holds O_i * 2^-E_i in fp16 and 2^E_i in part_scale, so its
// term is exp(lse_i - lse) * 2^E_i * (stored values).  Output bf16.
// fp16 partials: one thread per (row, head, 8 dims), so each part's O is one
// 16-byte load per thread (half the threads and loads of a 4-dim split,
// measured 0.65 us less per LingBot-frame call).
typedef _Float16 halfx8 __attribute__((__vector_size__(8 * sizeof(_Float16))));
typedef float floatx8 __attribute__((__vector_size__(8 * sizeof(float))));
typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
__global__ __launch_bounds__(256) void attn_merge16_kernel(int parts, int rows_heads, const _Float16* __restrict__ po,
                                                           const float* __restrict__ pscale,
                                                           const float* __restrict__ plse, uint16_t* __restrict__ o,
                                                           float* __restrict__ lse) {
  const int rh = blockIdx.x * 32 + (threadIdx.x >> 3);
  const int d8 = (threadIdx.x & 7) * 8;
  if (rh >= rows_heads) return;
  constexpr int B = 16;
  float m = -INFINITY, z = 0.f;
  floatx8 acc = {};
  for (int i0 = 0; i0 < parts; i0 += B) {
    float li[B], si[B];
    halfx8 oi[B];
#pragma unroll
    for (int j = 0; j < B; ++j) {
      const int i = i0 + j;
      const bool ok = i < parts;
      const size_t r = static_cast<size_t>(i) * rows_heads + rh;
      li[j] = ok ? plse[r] : -INFINITY;
      si[j] = ok ? pscale[r] : 0.f;
      oi[j] = ok ? *reinterpret_cast<const halfx8*>(po + r * D + d8) : halfx8{};
    }
    float mb = li[0];
#pragma unroll
    for (int j = 1; j < B; ++j) mb = fmaxf(mb, li[j]);
    if (mb == -INFINITY) continue;
    if (mb > m) {
      const float c = m == -INFINITY ? 0.f : __expf(m - mb);
      z *= c;
      acc *= c;
      m = mb;
    }
#pragma unroll
    for (int j = 0; j < B; ++j) {
      const float w = li[j] == -INFINITY ? 0.f : __expf(li[j] - m);
      z += w;
      const float ws = w * si[j];
      const floatx8 f = __builtin_convertvector(oi[j], floatx8);
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[k] = __builtin_fmaf(ws, f[k], acc[k]);
    }
  }
  floatx8 out;
#pragma unroll
  for (int k = 0; k < 8; ++k) out[k] = z > 0.f ? acc[k] / z : 0.f;
  *reinterpret_cast<bf16x8*>(o + static_cast<size_t>(rh) * D + d8) = __builtin_convertvector(out, bf16x8);
  if (lse && d8 == 0) lse[rh] = z > 0.f ? m + __logf(z) : -INFINITY;
}

}  // namespace

hipError_t launch_attn_merge(int dtype, int num_parts, int rows, int num_heads, const float* part_o,
                             const float* part_lse, void* o, float* lse, hipStream_t stream) {
  const int rh = rows * num_heads;
  if (rh == 0) return hipSuccess;
  const dim3 grid((rh + 15) / 16);
  if (dtype == 0)
    hipLaunchKernelGGL(attn_merge_kernel<uint16_t>, grid, dim3(256), 0, stream, num_parts, rh, part_o, part_lse,
                       static_cast<uint16_t*>(o), lse);
  else
    hipLaunchKernelGGL(attn_merge_kernel<float>, grid, dim3(256), 0, stream, num_parts, rh, part_o, part_lse,
                       static_cast<float*>(o), lse);
  return hipGetLastError();
}

hipError_t launch_attn_merge16(int num_parts, int rows, int num_heads, const _Float16* part_o16,
                               const float* part_scale, const float* part_lse, void* o, float* lse,
                               hipStream_t stream) {
  const int rh = rows * num_heads;
  if (rh == 0) return hipSuccess;
  const dim3 grid((rh + 31) / 32);
  hipLaunchKernelGGL(attn_merge16_kernel, grid, dim3(256), 0, stream, num_parts, rh, part_o16, part_scale, part_lse,
                     static_cast<uint16_t*>(o), lse);
  return hipGetLastError();
}

}  // namespace kvc
