// Roofline probes: the chip's measured dense bf16 matrix-core rate and HBM
// bandwidth, the denominators beside the published peaks, and the rate of the
// 512-row attention kernel's per-tile instruction mix on its own (declared in
// include/kvc_probe.h).  Each probe times a few launches of its kernel with
// HIP events on the given stream and blocks until they are done.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "handle.hpp"
#include "kvc.h"
#include "kvc_probe.h"

using kvc::fail;
using kvc::guarded;

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float floatx8 __attribute__((ext_vector_type(8)));

constexpr int kMfmaIters = 4096;
constexpr int kMfmaChains = 4;          // independent accumulators per wave
constexpr int kMfmaThreads = 1024;      // sixteen waves, four per SIMD
constexpr int kMfmaMaxBlocks = 1024;    // scratch sizing: at most this many compute units
constexpr int kMfmaPadFloats = 96 * 1024 / 4;  // 96 KiB of LDS: one workgroup per compute unit
constexpr double kMfmaFlop = 32.0 * 32.0 * 16.0 * 2.0;  // one v_mfma_f32_32x32x16_bf16

// One workgroup per compute unit (its LDS leaves no room for a second), every
// wave issuing kMfmaChains independent chains of 32x32x16 bf16 products from
// registers; the operands never change, so the products are all the kernel
// does.  One store per thread keeps the chains live.
__global__ __launch_bounds__(kMfmaThreads) void mfma_probe_kernel(float* out, float seed) {
  __shared__ float pad[kMfmaPadFloats];
  pad[threadIdx.x] = seed;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = static_cast<__bf16>(seed * static_cast<float>((threadIdx.x + i) & 7));
    b[i] = static_cast<__bf16>(seed - static_cast<float>(i));
  }
  floatx16 c[kMfmaChains];
#pragma unroll
  for (int j = 0; j < kMfmaChains; ++j) c[j] = floatx16{};
  for (int it = 0; it < kMfmaIters; ++it) {
#pragma unroll
    for (int j = 0; j < kMfmaChains; ++j) c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[j], 0, 0, 0);
  }
  __syncthreads();
  float s = pad[(threadIdx.x + 1) % kMfmaThreads];
#pragma unroll
  for (int j = 0; j < kMfmaChains; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += c[j][i];
  out[blockIdx.x * kMfmaThreads + threadIdx.x] = s;
}

// The 512-row attention kernel's work on one 64-key tile, per wave (two
// 32-row query blocks A and B, head dim 64), without global memory, table
// walk, masks or rare-path checks: a workgroup barrier; the tile's 8 K
// fragment reads from LDS; block A's 8 score products; 8 fenced groups of one
// of block B's score products and a four-element slice of block A's softmax
// (4 FMAs, 4 exponentials, 3 adds); block A's probabilities to bf16; the 8 V
// fragment reads; 8 fenced groups of one of block A's P V products and a slice
// of block B's softmax; block B's probabilities to bf16 and its 8 P V
// products.  Eight waves (two per SIMD) and the kernel's 96 KiB of LDS, so one
// workgroup per compute unit, as the kernel runs.
constexpr int kMixThreads = 512;
constexpr int kMixIters = 1024;
constexpr int kMixLdsFloats = 96 * 1024 / 4;
constexpr int kMixProducts = 32;  // per wave per tile

__device__ __forceinline__ bf16x8 mix_frag(const __bf16* base, int row, int chunk) {
  // 128-byte rows, 16-byte chunks XOR-swizzled by row as in the kernel
  const int sw = (row & 7) ^ ((row >> 3) & 1);
  return *reinterpret_cast<const bf16x8*>(base + row * 64 + ((chunk ^ sw) << 3));
}

__global__ __launch_bounds__(kMixThreads) void tile_mix_probe_kernel(float* out, float c) {
  __shared__ float lds[kMixLdsFloats];
  const int t = threadIdx.x;
  for (int i = t; i < kMixLdsFloats; i += kMixThreads) lds[i] = 0.001f * static_cast<float>(i & 127);
  const int lr = t & 31, lh = (t >> 5) & 1;
  bf16x8 qa[4], qb[4];
#pragma unroll
  for (int st = 0; st < 4; ++st)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      qa[st][i] = static_cast<__bf16>(0.01f * static_cast<float>((t + i + st) & 15));
      qb[st][i] = static_cast<__bf16>(0.01f * static_cast<float>((t + 2 * i - st) & 15));
    }
  const float m = 1.f;
  floatx16 oa0 = {}, oa1 = {}, ob0 = {}, ob1 = {};
  float la = 0.f, lb = 0.f;
  auto probs4 = [&](floatx16& sv, int b) {
#pragma unroll
    for (int r = 0; r < 4; ++r) sv[b + r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[b + r], c, -m));
    return (sv[b] + sv[b + 1]) + (sv[b + 2] + sv[b + 3]);
  };
  auto to_bf16 = [](const floatx16& sv, int base) {
    floatx8 f;
#pragma unroll
    for (int j = 0; j < 8; ++j) f[j] = sv[base + j];
    return __builtin_convertvector(f, bf16x8);
  };
  for (int it = 0; it < kMixIters; ++it) {
    const __bf16* lk = reinterpret_cast<const __bf16*>(lds) + (it % 6) * 8192;  // 6-tile ring, K then V^T
    __syncthreads();
    bf16x8 kf[8], vf[8];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      kf[st] = mix_frag(lk, lr, 2 * st + lh);
      kf[4 + st] = mix_frag(lk, 32 + lr, 2 * st + lh);
    }
    floatx16 sa0 = {}, sa1 = {}, sb0 = {}, sb1 = {};
#pragma unroll
    for (int st = 0; st < 4; ++st) sa0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[st], qa[st], sa0, 0, 0, 0);
#pragma unroll
    for (int st = 0; st < 4; ++st) sa1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[4 + st], qa[st], sa1, 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    float ps[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i < 4)
        sb0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i], qb[i], sb0, 0, 0, 0);
      else
        sb1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i], qb[i - 4], sb1, 0, 0, 0);
      ps[i] = probs4(i < 4 ? sa0 : sa1, 4 * (i & 3));
      __builtin_amdgcn_sched_barrier(0);
    }
    la += ((ps[0] + ps[1]) + (ps[2] + ps[3])) + ((ps[4] + ps[5]) + (ps[6] + ps[7]));
    bf16x8 pa[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) pa[q] = to_bf16(q < 2 ? sa0 : sa1, 8 * (q & 1));
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      vf[st] = mix_frag(lk + 4096, lr, 2 * st + lh);
      vf[4 + st] = mix_frag(lk + 4096, 32 + lr, 2 * st + lh);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i < 4)
        oa0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[i], pa[i], oa0, 0, 0, 0);
      else
        oa1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[i], pa[i - 4], oa1, 0, 0, 0);
      ps[i] = probs4(i < 4 ? sb0 : sb1, 4 * (i & 3));
      __builtin_amdgcn_sched_barrier(0);
    }
    lb += ((ps[0] + ps[1]) + (ps[2] + ps[3])) + ((ps[4] + ps[5]) + (ps[6] + ps[7]));
    bf16x8 pb[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) pb[q] = to_bf16(q < 2 ? sb0 : sb1, 8 * (q & 1));
#pragma unroll
    for (int q = 0; q < 4; ++q) ob0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[q], pb[q], ob0, 0, 0, 0);
#pragma unroll
    for (int q = 0; q < 4; ++q) ob1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[4 + q], pb[q], ob1, 0, 0, 0);
  }
  float r = la + lb;
#pragma unroll
  for (int i = 0; i < 16; ++i) r += oa0[i] + oa1[i] + ob0[i] + ob1[i];
  out[blockIdx.x * kMixThreads + t] = r;
}

constexpr int kCopyThreads = 256;

// Streaming copy, 16 bytes per thread per step (grid-stride).
__global__ __launch_bounds__(kCopyThreads) void copy_probe_kernel(const u32x4* __restrict__ src,
                                                                  u32x4* __restrict__ dst, size_t n) {
  const size_t stride = static_cast<size_t>(gridDim.x) * kCopyThreads;
  for (size_t i = static_cast<size_t>(blockIdx.x) * kCopyThreads + threadIdx.x; i < n; i += stride)
    dst[i] = __builtin_nontemporal_load(src + i);
}

// Streaming read: every thread folds its 16-byte loads into one word and
// stores it once (out holds one word per thread of the grid).
__global__ __launch_bounds__(kCopyThreads) void read_probe_kernel(const u32x4* __restrict__ src, size_t n,
                                                                  uint32_t* __restrict__ out) {
  const size_t stride = static_cast<size_t>(gridDim.x) * kCopyThreads;
  u32x4 acc = {0u, 0u, 0u, 0u};
  const size_t t = static_cast<size_t>(blockIdx.x) * kCopyThreads + threadIdx.x;
  for (size_t i = t; i < n; i += stride) acc ^= __builtin_nontemporal_load(src + i);
  out[t] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

constexpr int kStreamBlocks = 256 * 8;  // eight workgroups per compute unit
constexpr int kReps = 5;

// Times kReps launches of `launch` after one untimed launch; milliseconds per launch.
template <class F>
int time_launches(hipStream_t st, F&& launch, double* ms_per) {
  hipEvent_t e0 = nullptr, e1 = nullptr;
  int status = KVC_OK;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) {
    status = fail(KVC_ERR_DEVICE, "probe: hipEventCreate failed");
  } else {
    launch();
    hipError_t e = hipEventRecord(e0, st);
    for (int r = 0; r < kReps; ++r) launch();
    if (e == hipSuccess) e = hipEventRecord(e1, st);
    if (e == hipSuccess) e = hipGetLastError();
    if (e == hipSuccess) e = hipEventSynchronize(e1);
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
    if (e != hipSuccess)
      status = fail(KVC_ERR_DEVICE, "probe: %s", hipGetErrorString(e));
    else
      *ms_per = static_cast<double>(ms) / kReps;
  }
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  return status;
}

}  // namespace

extern "C" {

size_t kvc_probe_scratch_bytes(void) {
  return std::max(static_cast<size_t>(kMfmaMaxBlocks) * kMfmaThreads * sizeof(float),
                  static_cast<size_t>(kStreamBlocks) * kCopyThreads * sizeof(uint32_t));
}

int kvc_probe_mfma_bf16(void* scratch, size_t scratch_bytes, kvc_stream_t stream, double* tflops) {
  return guarded("kvc_probe_mfma_bf16", [&] {
    if (!scratch || !tflops) return fail(KVC_ERR_INVALID_ARGUMENT, "NULL argument");
    if (scratch_bytes < kvc_probe_scratch_bytes())
      return fail(KVC_ERR_BUFFER_TOO_SMALL, "scratch needs %zu bytes", kvc_probe_scratch_bytes());
    const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      return fail(KVC_ERR_DEVICE, "probe: cannot read the compute-unit count");
    const int blocks = std::min(cus, kMfmaMaxBlocks);
    double ms = 0.0;
    const int s = time_launches(st, [&] {
      hipLaunchKernelGGL(mfma_probe_kernel, dim3(blocks), dim3(kMfmaThreads), 0, st, static_cast<float*>(scratch),
                         0.5f);
    }, &ms);
    if (s) return s;
    const double flop = kMfmaFlop * kMfmaChains * kMfmaIters * (kMfmaThreads / 64) * blocks;
    *tflops = flop / (ms * 1e-3) / 1e12;
    return static_cast<int>(KVC_OK);
  });
}

int kvc_probe_tile_mix(void* scratch, size_t scratch_bytes, kvc_stream_t stream, double* tflops) {
  return guarded("kvc_probe_tile_mix", [&] {
    if (!scratch || !tflops) return fail(KVC_ERR_INVALID_ARGUMENT, "NULL argument");
    if (scratch_bytes < kvc_probe_scratch_bytes())
      return fail(KVC_ERR_BUFFER_TOO_SMALL, "scratch needs %zu bytes", kvc_probe_scratch_bytes());
    const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      return fail(KVC_ERR_DEVICE, "probe: cannot read the compute-unit count");
    const int blocks = std::min(cus, kMfmaMaxBlocks);  // scratch holds kMfmaThreads >= kMixThreads floats per block
    double ms = 0.0;
    const int s = time_launches(st, [&] {
      hipLaunchKernelGGL(tile_mix_probe_kernel, dim3(blocks), dim3(kMixThreads), 0, st, static_cast<float*>(scratch),
                         0.18033688f);
    }, &ms);
    if (s) return s;
    const double flop = kMfmaFlop * kMixProducts * kMixIters * (kMixThreads / 64) * blocks;
    *tflops = flop / (ms * 1e-3) / 1e12;
    return static_cast<int>(KVC_OK);
  });
}

int kvc_probe_hbm(const void* src, void* dst, size_t bytes, void* scratch, size_t scratch_bytes,
                  kvc_stream_t stream, double* read_gbs, double* copy_gbs) {
  return guarded("kvc_probe_hbm", [&] {
    if (!src || !dst || !scratch || !read_gbs || !copy_gbs) return fail(KVC_ERR_INVALID_ARGUMENT, "NULL argument");
    if (bytes < 16 || bytes % 16 || ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15))
      return fail(KVC_ERR_INVALID_ARGUMENT, "bytes must be a positive multiple of 16 and buffers 16-byte aligned");
    if (scratch_bytes < kvc_probe_scratch_bytes())
      return fail(KVC_ERR_BUFFER_TOO_SMALL, "scratch needs %zu bytes", kvc_probe_scratch_bytes());
    const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const size_t n = bytes / 16;
    double ms = 0.0;
    int s = time_launches(st, [&] {
      hipLaunchKernelGGL(read_probe_kernel, dim3(kStreamBlocks), dim3(kCopyThreads), 0, st,
                         static_cast<const u32x4*>(src), n, static_cast<uint32_t*>(scratch));
    }, &ms);
    if (s) return s;
    *read_gbs = static_cast<double>(bytes) / (ms * 1e-3) / 1e9;
    s = time_launches(st, [&] {
      hipLaunchKernelGGL(copy_probe_kernel, dim3(kStreamBlocks), dim3(kCopyThreads), 0, st,
                         static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), n);
    }, &ms);
    if (s) return s;
    *copy_gbs = 2.0 * static_cast<double>(bytes) / (ms * 1e-3) / 1e9;
    return static_cast<int>(KVC_OK);
  });
}

}  // extern "C"
