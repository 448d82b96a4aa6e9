// Merge of split-key partial attention results.
//
// When a sequence's key range is split across workgroups, each part yields an
// output normalised over its own keys and the log-sum-exp of its scaled
// scores.  The full result is the log-sum-exp-weighted average of the parts:
//   lse = log sum_i exp(lse_i),   O = sum_i exp(lse_i - lse) O_i.
// Parts with lse_i = -inf (no keys) carry zero weight; if every part is empty
// the output is 0 and lse is -inf.
//
// One thread per (row, head, dim); 64 consecutive threads read one part's
// 256-byte row, so every access is coalesced, and each thread keeps eight
// parts' loads in flight at once.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernels.hpp"

namespace kvc {
namespace {

constexpr int D = kHeadDim;

template <typename T>
__device__ __forceinline__ void store_out(T* o, size_t i, float v);
template <>
__device__ __forceinline__ void store_out<uint16_t>(uint16_t* o, size_t i, float v) {
  const __bf16 b = static_cast<__bf16>(v);
  o[i] = __builtin_bit_cast(uint16_t, b);
}
template <>
__device__ __forceinline__ void store_out<float>(float* o, size_t i, float v) {
  o[i] = v;
}

template <typename T>
__global__ __launch_bounds__(256) void attn_merge_kernel(int parts, int rows_heads, const float* __restrict__ po,
                                                         const float* __restrict__ plse, T* __restrict__ o,
                                                         float* __restrict__ lse) {
  const int rh = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int d = threadIdx.x & 63;
  if (rh >= rows_heads) return;
  // Parts are consumed in batches of 8 whose loads are all issued together;
  // the running maximum m keeps the weights finite across batches.
  constexpr int B = 8;
  float m = -INFINITY, z = 0.f, acc = 0.f;
  for (int i0 = 0; i0 < parts; i0 += B) {
    float li[B], oi[B];
#pragma unroll
    for (int j = 0; j < B; ++j) {
      const int i = i0 + j;
      const bool ok = i < parts;
      li[j] = ok ? plse[static_cast<size_t>(i) * rows_heads + rh] : -INFINITY;
      oi[j] = ok ? po[(static_cast<size_t>(i) * rows_heads + rh) * D + d] : 0.f;
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
      acc = __builtin_fmaf(w, oi[j], acc);
    }
  }
  const float out = z > 0.f ? acc / z : 0.f;
  store_out<T>(o, static_cast<size_t>(rh) * D + d, out);
  if (lse && d == 0) lse[rh] = z > 0.f ? m + __logf(z) : -INFINITY;
}

}  // namespace

hipError_t launch_attn_merge(int dtype, int num_parts, int rows, int num_heads, const float* part_o,
                             const float* part_lse, void* o, float* lse, hipStream_t stream) {
  const int rh = rows * num_heads;
  if (rh == 0) return hipSuccess;
  const dim3 grid((rh + 3) / 4);
  if (dtype == 0)
    hipLaunchKernelGGL(attn_merge_kernel<uint16_t>, grid, dim3(256), 0, stream, num_parts, rh, part_o, part_lse,
                       static_cast<uint16_t*>(o), lse);
  else
    hipLaunchKernelGGL(attn_merge_kernel<float>, grid, dim3(256), 0, stream, num_parts, rh, part_o, part_lse,
                       static_cast<float*>(o), lse);
  return hipGetLastError();
}

}  // namespace kvc
