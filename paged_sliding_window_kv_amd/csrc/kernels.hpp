// Internal launch interface between the C ABI and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace kvc {

// V pools store each [dim][slot] row with the middle two 4-slot groups of
// every 16-slot group swapped: slot s lives at element v_slot_pos(s).  The
// map is its own inverse.  (It makes a 16-byte chunk of a row one operand
// fragment of the bf16 kernel's P*V product.)
__host__ __device__ constexpr int v_slot_pos(int s) { return (s & ~15) | (s & 3) | ((s & 4) << 1) | ((s & 8) >> 1); }

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
  void* k_exp;            // FP8 caches: row exponents [pages][H][P] (int8), after the codes
  void* v_exp;
  void* k_copy;           // null, or [T][H][d] activations: the unit's K/V rows as read, copied here too
  void* v_copy;
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
  float* part_o;          // [splits][total_q][H][d] when splits > 1 (fp32 kernel)
  float* part_lse;        // [splits][total_q][H]
  // bf16/FP8 kernels: partial O in fp16 as O * 2^-E (E >= 0, so that every
  // value stays within fp16 range), with 2^E per (split, row, head).
  _Float16* part_o16;     // [splits][total_q][H][d]
  float* part_scale;      // [splits][total_q][H]
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

// Most table entries and sequences passed by value in the kernel arguments.
// Each entry packs page id (low 20 bits) and valid length (high 12 bits);
// with the parameters above the argument block stays under 3 KiB.
constexpr int kMaxInlinePages = 640;
constexpr int kMaxInlineSeqs = 16;
constexpr int kInlinePidBits = 20;
constexpr int kInlineMaxPid = (1 << kInlinePidBits) - 1;

// Paged attention whose tables travel in the kernel arguments: sequence s
// has queries [qo[s], qo[s+1]) and entries [kv[s], kv[s+1]) of `entries`.
struct AttnParamsInline {
  AttnParams base;
  int32_t num_entries;
  int32_t qo[kMaxInlineSeqs + 1];
  int32_t kv[kMaxInlineSeqs + 1];
  uint32_t entries[kMaxInlinePages];
};

// Table access shared by the attention kernels, for both table sources.
__host__ __device__ __forceinline__ const AttnParams& attn_base(const AttnParams& p) { return p; }
__host__ __device__ __forceinline__ const AttnParams& attn_base(const AttnParamsInline& p) { return p.base; }

// Device tables are read through the constant address space: the reads are
// wave-uniform, so they become scalar loads, which leave the vector-memory
// wait counts of the attention kernels to the K/V tile loads alone.
typedef const __attribute__((address_space(4))) int32_t const_i32;
__device__ __forceinline__ int32_t ld_const(const int32_t* p, int i) {
  return reinterpret_cast<const_i32*>(reinterpret_cast<uintptr_t>(p))[i];
}

__device__ __forceinline__ void attn_seq(const AttnParams& p, int seq, int& q0, int& qn, int& e0, int& en) {
  q0 = ld_const(p.qo_indptr, seq);
  qn = ld_const(p.qo_indptr, seq + 1) - q0;
  e0 = ld_const(p.kv_indptr, seq);
  en = ld_const(p.kv_indptr, seq + 1) - e0;
}
__device__ __forceinline__ void attn_seq(const AttnParamsInline& p, int seq, int& q0, int& qn, int& e0, int& en) {
  q0 = p.qo[seq];
  qn = p.qo[seq + 1] - q0;
  e0 = p.kv[seq];
  en = p.kv[seq + 1] - e0;
}

// Workgroup index -> (group, query tile).  The dispatcher hands workgroups to
// the eight XCDs round-robin by index, so XCD x runs indices x, x+8, x+16, ...
// The i-th of those takes query tile i % q_tiles of group 8 * (i / q_tiles) + x:
// all query tiles of one (sequence, head, split) group run on one XCD, one
// after the other, so the workgroups an XCD holds at a time read the key
// ranges of one or two groups, which its L2 then serves to all of them.
// groups_padded (a multiple of 8) times q_tiles workgroups cover every pair;
// groups at or past p.groups are padding.
__device__ __forceinline__ void attn_tile_of(const AttnParams& p, int wg, int& g, int& qt) {
  const int x = wg & 7, i = wg >> 3;
  qt = i % p.q_tiles;
  g = (i / p.q_tiles) * 8 + x;
}

// Page id and valid length of table entry e; invalid ids and lengths give 0.
__device__ __forceinline__ void attn_entry(const AttnParams& p, int e, int& pid, int& len) {
  pid = ld_const(p.page_ids, e);
  len = ld_const(p.page_lens, e);
  len = len < 0 ? 0 : (len > p.page_size ? p.page_size : len);
  if (pid < 0 || pid >= p.num_pool_pages) len = 0;
}
__device__ __forceinline__ void attn_entry(const AttnParamsInline& p, int e, int& pid, int& len) {
  const uint32_t w = p.entries[e];
  pid = static_cast<int>(w & kInlineMaxPid);
  len = static_cast<int>(w >> kInlinePidBits);
  len = len > p.base.page_size ? p.base.page_size : len;
  if (pid >= p.base.num_pool_pages) len = 0;
}

// Rows of queries one workgroup of the bf16 kernel covers.
int attn_bf16_rows_per_tile(int waves);
hipError_t launch_attn_bf16(const AttnParams& p, int waves, hipStream_t stream);
hipError_t launch_attn_bf16(const AttnParamsInline& p, int waves, hipStream_t stream);
// FP8 (E4M3) pools with row exponents; q and o bf16.  Same row tiling as the bf16 kernel.
hipError_t launch_attn_fp8kv(const AttnParams& p, int waves, hipStream_t stream);
hipError_t launch_attn_fp8kv(const AttnParamsInline& p, int waves, hipStream_t stream);
int attn_f32_rows_per_tile();
hipError_t launch_attn_f32(const AttnParams& p, hipStream_t stream);
hipError_t launch_attn_f32(const AttnParamsInline& p, hipStream_t stream);

hipError_t launch_attn_merge(int dtype, int num_parts, int rows, int num_heads, const float* part_o,
                             const float* part_lse, void* o, float* lse, hipStream_t stream);
// Partials in the fp16 form (part_o16, part_scale); o is bf16.
hipError_t launch_attn_merge16(int num_parts, int rows, int num_heads, const _Float16* part_o16,
                               const float* part_scale, const float* part_lse, void* o, float* lse,
                               hipStream_t stream);

}  // namespace kvc
