// KV-append scatter: one unit's K/V rows into its pages.
// V rows are written in the pool's slot order (v_slot_pos).
//
// "LingBot-Map Paged KV Cache", section 2: a frame's 256 patch tokens fill one
// page of the patch stream and its 6 special tokens are packed into the
// current special page.  "vLLM-Omni RFC #2727", section 3.3: the chunk step
// appends the chunk's KV to the cache.
//
// Pure data movement, bound by HBM bandwidth.  Each workgroup moves a tile of
// 64 consecutive tokens of one head.  K rows are copied with 16-byte vector
// accesses (source and destination rows are both contiguous).  V is stored
// transposed in the pool ([dim][slot] per page and head) so that the
// attention kernel reads it as the row operand of its P*V product; the tile
// goes through LDS and leaves as 16-byte runs of 8 (bf16) or 4 (fp32)
// consecutive slots.  When AppendParams::k_copy is set (windowed mode), every
// K and V chunk read is also written unchanged to the copy buffers, at its
// source offset.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernels.hpp"

namespace kvc {
namespace {

constexpr int kTile = 64;
// One thread per 16-byte chunk of a tile's K rows (and of its V rows), so each
// thread issues its loads once and no thread loops over memory round trips:
// 512 threads for bf16, 1024 for fp32.
template <typename T>
constexpr int append_threads() {
  return kTile * (kHeadDim * static_cast<int>(sizeof(T)) / 16);
}

struct Dest {
  int32_t page;
  int32_t slot;
};

__device__ __forceinline__ Dest dest_of(const AppendParams& p, int tok) {
  if (tok < p.patch_tokens) return {p.unit_pages[tok / p.page_size], tok % p.page_size};
  const int j = tok - p.patch_tokens;
  if (j < p.special_count0) return {p.special_page0, p.special_slot0 + j};
  return {p.special_page1, j - p.special_count0};
}

// T: element type (uint16_t bf16 pattern or float).  VEC elements per 16 bytes.
template <typename T>
__global__ __launch_bounds__(append_threads<T>()) void kv_append_kernel(const AppendParams p) {
  constexpr int kThreads = append_threads<T>();
  constexpr int VEC = 16 / sizeof(T);
  constexpr int D = kHeadDim;
  constexpr int CHUNKS = D / VEC;  // 16-byte chunks per token row
  using V16 = uint4;
  __shared__ T vt[kTile][D + VEC];  // padded rows

  const int h = blockIdx.y;
  const int H = p.num_heads;
  const int P = p.page_size;
  const int patch_tiles = (p.patch_tokens + kTile - 1) / kTile;
  int tok0, ntok;
  if (static_cast<int>(blockIdx.x) < patch_tiles) {
    tok0 = blockIdx.x * kTile;
    ntok = min(kTile, p.patch_tokens - tok0);
  } else {
    const int st = blockIdx.x - patch_tiles;
    tok0 = p.patch_tokens + st * kTile;
    ntok = min(kTile, p.patch_tokens + p.special_tokens - tok0);
  }
  if (ntok <= 0) return;

  const T* ksrc = static_cast<const T*>(p.k_src);
  const T* vsrc = static_cast<const T*>(p.v_src);
  T* kpool = static_cast<T*>(p.k_pool);
  T* vpool = static_cast<T*>(p.v_pool);

  // K: contiguous rows, 16-byte copies; V: rows staged in LDS.
  for (int c = threadIdx.x; c < ntok * CHUNKS; c += kThreads) {
    const int t = c / CHUNKS, ch = c % CHUNKS;
    const int tok = tok0 + t;
    const size_t src = (static_cast<size_t>(tok) * H + h) * D + ch * VEC;
    const Dest dd = dest_of(p, tok);
    const size_t dst = ((static_cast<size_t>(dd.page) * H + h) * P + dd.slot) * D + ch * VEC;
    const V16 k = *reinterpret_cast<const V16*>(ksrc + src);
    const V16 v = *reinterpret_cast<const V16*>(vsrc + src);
    *reinterpret_cast<V16*>(kpool + dst) = k;
    if (p.k_copy) {  // workgroup-uniform
      *reinterpret_cast<V16*>(static_cast<T*>(p.k_copy) + src) = k;
      *reinterpret_cast<V16*>(static_cast<T*>(p.v_copy) + src) = v;
    }
    const T* ve = reinterpret_cast<const T*>(&v);
#pragma unroll
    for (int e = 0; e < VEC; ++e) vt[t][ch * VEC + e] = ve[e];
  }
  __syncthreads();

  // Fast path: the whole tile lands on consecutive slots of one page.
  const Dest first = dest_of(p, tok0);
  const Dest last = dest_of(p, tok0 + ntok - 1);
  const bool run = first.page == last.page && last.slot - first.slot == ntok - 1 && (first.slot % 16) == 0 &&
                   (ntok % 16) == 0;
  if (run) {
    const int groups = ntok / VEC;  // 16-byte runs per dim row
    for (int c = threadIdx.x; c < D * groups; c += kThreads) {
      const int d = c / groups, g = c % groups;
      V16 out;
      T* oe = reinterpret_cast<T*>(&out);
      // element g*VEC + e of the run holds slot v_slot_pos(g*VEC + e) (runs start 16-aligned)
#pragma unroll
      for (int e = 0; e < VEC; ++e) oe[e] = vt[v_slot_pos(g * VEC + e)][d];
      const size_t dst = ((static_cast<size_t>(first.page) * H + h) * D + d) * P + first.slot + g * VEC;
      *reinterpret_cast<V16*>(vpool + dst) = out;
    }
  } else {
    for (int c = threadIdx.x; c < D * ntok; c += kThreads) {
      const int d = c / ntok, t = c % ntok;
      const Dest dd = dest_of(p, tok0 + t);
      const size_t dst = ((static_cast<size_t>(dd.page) * H + h) * D + d) * P + v_slot_pos(dd.slot);
      vpool[dst] = vt[t][d];
    }
  }
}

// ---------------------------------------------------------------------------
// FP8 caches ("vLLM-Omni RFC #2727", section 3.4, item 5: KV cache FP8).
// Each (token, head) row of d = 64 bf16 values becomes 64 OCP E4M3 codes and
// one int8 exponent e: e is the smallest integer in [-127, 127] with
// max|x| <= 448 * 2^e, and each code is x / 2^e rounded to the nearest E4M3
// value, ties to the even code.  K and V rows both go slot-major into
// their pools; the exponents go to [page][head][slot] after the codes.
// ---------------------------------------------------------------------------

// Smallest e in [-127, 127] with amax <= 448 * 2^e (-127 for amax = 0).
__device__ __forceinline__ int fp8_row_exponent(float amax) {
  if (amax == 0.f) return -127;
  int fe;
  const float fm = frexpf(amax, &fe);  // amax = fm * 2^fe, fm in [0.5, 1)
  const int E = fe - 1;
  const int e = (2.f * fm <= 1.75f) ? E - 8 : E - 7;
  return max(-127, min(127, e));
}

// Nearest E4M3 code to y (|y| <= 448), ties to the even code.
__device__ __forceinline__ uint32_t e4m3_rne(float y) {
  const uint32_t b = __float_as_uint(y);
  const uint32_t sign = (b >> 24) & 0x80u;
  const uint32_t a = b & 0x7fffffffu;
  if (a < 0x3C800000u) {  // |y| < 2^-6: subnormal codes, steps of 2^-9 (the product is exact)
    const float m = rintf(__uint_as_float(a) * 512.f);
    return sign | static_cast<uint32_t>(m);  // 8 is the smallest normal, code 0x08
  }
  // Normal: keep 3 mantissa bits, round half to even; a carry moves into the
  // exponent field.  Exponent bias 127 -> 7 is a subtraction of 120 << 3.
  const uint32_t r = (a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20;
  return sign | (r - (120u << 3));
}

constexpr int kFp8RowThreads = 8;  // threads per (token, head) row, 8 values each
constexpr int kFp8Threads = 2 * kTile * kFp8RowThreads;  // every K and V row of a tile at once

__global__ __launch_bounds__(kFp8Threads) void kv_append_fp8_kernel(const AppendParams p) {
  constexpr int kThreads = kFp8Threads;
  constexpr int D = kHeadDim;
  const int h = blockIdx.y;
  const int H = p.num_heads;
  const int P = p.page_size;
  const int patch_tiles = (p.patch_tokens + kTile - 1) / kTile;
  int tok0, ntok;
  if (static_cast<int>(blockIdx.x) < patch_tiles) {
    tok0 = blockIdx.x * kTile;
    ntok = min(kTile, p.patch_tokens - tok0);
  } else {
    const int st = blockIdx.x - patch_tiles;
    tok0 = p.patch_tokens + st * kTile;
    ntok = min(kTile, p.patch_tokens + p.special_tokens - tok0);
  }
  if (ntok <= 0) return;
  const int lane8 = threadIdx.x & (kFp8RowThreads - 1);
  // Rows are processed by aligned groups of 8 lanes; every lane of a wave runs
  // the same number of iterations, so the group reductions below see all 8.
  for (int it = threadIdx.x / kFp8RowThreads; it < 2 * kTile; it += kThreads / kFp8RowThreads) {
    const int t = it % kTile;
    const bool is_v = it >= kTile;
    const bool valid = t < ntok;
    const int tok = tok0 + (valid ? t : 0);
    const uint16_t* src = static_cast<const uint16_t*>(is_v ? p.v_src : p.k_src) +
                          (static_cast<size_t>(tok) * H + h) * D + lane8 * 8;
    uint4 raw = {0u, 0u, 0u, 0u};
    if (valid) {
      raw = *reinterpret_cast<const uint4*>(src);
      if (p.k_copy) {  // the row as read, into the copy at the same offset
        const size_t off = (static_cast<size_t>(tok) * H + h) * D + lane8 * 8;
        *reinterpret_cast<uint4*>(static_cast<uint16_t*>(is_v ? p.v_copy : p.k_copy) + off) = raw;
      }
    }
    float x[8];
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
#pragma unroll
    for (int m = 1; m < kFp8RowThreads; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m, kFp8RowThreads));
    const int e = fp8_row_exponent(amax);
    uint32_t c[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i >> 2] |= e4m3_rne(ldexpf(x[i], -e)) << (8 * (i & 3));
    if (!valid) continue;
    const Dest dd = dest_of(p, tok);
    const size_t row = (static_cast<size_t>(dd.page) * H + h) * P + dd.slot;
    uint8_t* pool = static_cast<uint8_t*>(is_v ? p.v_pool : p.k_pool);
    *reinterpret_cast<uint2*>(pool + row * D + lane8 * 8) = make_uint2(c[0], c[1]);
    if (lane8 == 0) static_cast<int8_t*>(is_v ? p.v_exp : p.k_exp)[row] = static_cast<int8_t>(e);
  }
}

}  // namespace

hipError_t launch_kv_append(const AppendParams& p, int dtype, hipStream_t stream) {
  const int tiles = (p.patch_tokens + kTile - 1) / kTile + (p.special_tokens + kTile - 1) / kTile;
  if (tiles == 0) return hipSuccess;
  dim3 grid(tiles, p.num_heads);
  if (dtype == 0)
    hipLaunchKernelGGL(kv_append_kernel<uint16_t>, grid, dim3(append_threads<uint16_t>()), 0, stream, p);
  else if (dtype == 1)
    hipLaunchKernelGGL(kv_append_kernel<float>, grid, dim3(append_threads<float>()), 0, stream, p);
  else
    hipLaunchKernelGGL(kv_append_fp8_kernel, grid, dim3(kFp8Threads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace kvc
