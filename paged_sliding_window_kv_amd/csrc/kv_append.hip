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
// consecutive slots.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernels.hpp"

namespace kvc {
namespace {

constexpr int kTile = 64;
constexpr int kThreads = 256;

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
__global__ __launch_bounds__(kThreads) void kv_append_kernel(const AppendParams p) {
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
    *reinterpret_cast<V16*>(kpool + dst) = *reinterpret_cast<const V16*>(ksrc + src);
    const V16 v = *reinterpret_cast<const V16*>(vsrc + src);
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

}  // namespace

hipError_t launch_kv_append(const AppendParams& p, int dtype, hipStream_t stream) {
  const int tiles = (p.patch_tokens + kTile - 1) / kTile + (p.special_tokens + kTile - 1) / kTile;
  if (tiles == 0) return hipSuccess;
  dim3 grid(tiles, p.num_heads);
  if (dtype == 0)
    hipLaunchKernelGGL(kv_append_kernel<uint16_t>, grid, dim3(kThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(kv_append_kernel<float>, grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace kvc
