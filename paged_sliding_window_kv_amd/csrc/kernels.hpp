// Internal launch interface between the C ABI and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace kvc {

// Most pages one unit may span (one chunk of 8 VGGT frames is 43 pages).
constexpr int kMaxUnitPages = 256;
// Head dim and key tile of the device kernels.
constexpr int kHeadDim = 64;
constexpr int kKeyTile = 64;

// Scatter of one unit's K/V rows into its pages.  Passed by value so that the
// launch needs no device-side table.
struct AppendParams {
  const void* k_src;  // [T][H][d], T = patch_tokens + special_tokens
  const void* v_src;
  void* k_pool;       // [pages][H][P][d]
  void* v_pool;       // [pages][H][d][P]
  int32_t num_heads;
  int32_t page_size;
  int32_t patch_tokens;
  int32_t special_tokens;
  int32_t special_page0;
  int32_t special_slot0;
  int32_t special_count0;
  int32_t special_page1;
  int32_t num_unit_pages;
  int32_t unit_pages[kMaxUnitPages];
};

hipError_t launch_kv_append(const AppendParams& p, int dtype, hipStream_t stream);

// Paged attention over a device page table.
struct AttnParams {
  const void* q;          // [total_q][H][d]
  const void* k_pool;
  const void* v_pool;
  void* o;                // [total_q][H][d]
  float* lse;             // [total_q][H] or null
  float* part_o;          // [splits][total_q][H][d] when splits > 1
  float* part_lse;        // [splits][total_q][H]
  const int32_t* qo_indptr;
  const int32_t* kv_indptr;
  const int32_t* page_ids;
  const int32_t* page_lens;
  int32_t num_heads;
  int32_t page_size;
  int32_t num_pool_pages;
  int32_t num_seqs;
  int32_t total_q;
  int32_t q_tiles;        // query tiles per sequence (grid sizing)
  int32_t num_splits;
  int32_t groups;         // num_seqs * num_heads * num_splits
  int32_t groups_padded;  // groups rounded up to a multiple of 8 (XCD count)
  float sm_scale;
  float scale_log2;       // sm_scale * log2(e)
};

// Rows of queries one workgroup of the bf16 kernel covers.
int attn_bf16_rows_per_tile(int waves);
hipError_t launch_attn_bf16(const AttnParams& p, int waves, hipStream_t stream);
int attn_f32_rows_per_tile();
hipError_t launch_attn_f32(const AttnParams& p, hipStream_t stream);

hipError_t launch_attn_merge(int dtype, int num_parts, int rows, int num_heads, const float* part_o,
                             const float* part_lse, void* o, float* lse, hipStream_t stream);

}  // namespace kvc
