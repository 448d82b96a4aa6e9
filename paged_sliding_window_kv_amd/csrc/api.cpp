// C ABI of libkvc.so (declared in include/kvc.h).
//
// Every extern "C" entry point runs its body inside kvc::guarded(), so no C++
// exception crosses the boundary; appends plan on the host, launch, and only
// then commit, so a failed launch leaves the cache as it was.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "handle.hpp"
#include "kernels.hpp"
#include "kvc.h"
#include "page_cache.hpp"
#include "subset.hpp"

namespace kvc {

namespace {
thread_local char g_last_error[512] = "";
// Measurement hook (kvc_set_kernel_events): recorded on the launch stream
// right before and right after each attention kernel (before the merge of
// split partials).
thread_local hipEvent_t g_kernel_start = nullptr;
thread_local hipEvent_t g_kernel_done = nullptr;
}  // namespace

int fail(int status, const char* fmt, ...) noexcept {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return status;
}

TableRing::~TableRing() {
  for (int i = 0; i < kSlots; ++i)
    if (done[i]) {
      if (in_flight[i]) (void)hipEventSynchronize(done[i]);
      (void)hipEventDestroy(done[i]);
    }
  if (host) (void)hipHostFree(host);
}

int32_t* TableRing::acquire(size_t words, int* slot) {
  if (!host || words > slot_words) {
    // first use, or a longer table than the slots hold: (re)size, after every
    // copy from the old slots has completed
    for (int i = 0; i < kSlots; ++i)
      if (in_flight[i]) {
        if (hipEventSynchronize(done[i]) != hipSuccess) {
          fail(KVC_ERR_DEVICE, "table staging: waiting for an earlier copy failed");
          return nullptr;
        }
        in_flight[i] = false;
      }
    if (host) (void)hipHostFree(host);
    host = nullptr;
    const size_t w = std::max<size_t>(words, 1024);
    if (hipHostMalloc(reinterpret_cast<void**>(&host), kSlots * w * sizeof(int32_t), hipHostMallocDefault) !=
        hipSuccess) {
      host = nullptr;
      fail(KVC_ERR_DEVICE, "table staging: hipHostMalloc of %zu bytes failed", kSlots * w * sizeof(int32_t));
      return nullptr;
    }
    slot_words = w;
    for (int i = 0; i < kSlots; ++i)
      if (!done[i] && hipEventCreateWithFlags(&done[i], hipEventDisableTiming) != hipSuccess) {
        done[i] = nullptr;
        fail(KVC_ERR_DEVICE, "table staging: hipEventCreate failed");
        return nullptr;
      }
  }
  const int s = next;
  if (in_flight[s]) {
    if (hipEventSynchronize(done[s]) != hipSuccess) {
      fail(KVC_ERR_DEVICE, "table staging: waiting for an earlier copy failed");
      return nullptr;
    }
    in_flight[s] = false;
  }
  next = (next + 1) % kSlots;
  *slot = s;
  return host + static_cast<size_t>(s) * slot_words;
}

}  // namespace kvc

using kvc::fail;
using kvc::guarded;

namespace {

size_t elem_size(int dtype) { return dtype == KVC_DTYPE_BF16 ? 2 : dtype == KVC_DTYPE_F32 ? 4 : 1; }

// Bytes of one pool: elements, plus the row exponents of FP8 pools.
size_t pool_bytes(const kvc_config& c, int32_t pages) {
  const size_t rows = static_cast<size_t>(pages) * c.num_heads * c.page_size;
  return rows * c.head_dim * elem_size(c.dtype) + (c.dtype == KVC_DTYPE_FP8_E4M3 ? rows : 0);
}

bool device_shapes_ok(const kvc_config& c) {
  return c.head_dim == kvc::kHeadDim && c.page_size % kvc::kKeyTile == 0;
}

constexpr int kXcds = 8;

int choose_waves(const paged_attn_args& a) {
  // Up to 256 query rows: one 32-row block per 32 rows (two waves each), all
  // in one workgroup, so each key tile is read once per split.  Beyond that,
  // 272-row workgroups (eight blocks plus a 16-row extra block, returned as 9)
  // when they need at least 10% fewer query tiles than 256-row ones (a frame of
  // 262 queries: one tile instead of two); otherwise 256-row workgroups, whose
  // per-step work is even across the waves (measured 9% faster on 10,992-row
  // chunks, where the tile counts are 41 and 43).  Above 1,024 queries, bf16
  // and FP8 pages take 512-row tiles (returned as 10: eight waves, two 32-row
  // blocks each).
  const long q = a.max_qo_len;
  if (a.dtype != KVC_DTYPE_F32 && q > 1024) return 10;
  if (q <= 256) return std::max(1, static_cast<int>((q + 31) / 32));
  const long t272 = (q + 271) / 272, t256 = (q + 255) / 256;
  return 10 * t256 >= 11 * t272 ? 9 : 8;
}

int rows_per_tile(const paged_attn_args& a) {
  return a.dtype != KVC_DTYPE_F32 ? kvc::attn_bf16_rows_per_tile(choose_waves(a)) : kvc::attn_f32_rows_per_tile();
}

// Workgroups the chip holds at once: one bf16/FP8 workgroup per compute unit
// (each uses more than half of a unit's LDS), several one-wave fp32 ones.
long workgroup_slots(const paged_attn_args& a) { return a.dtype != KVC_DTYPE_F32 ? 256 : 512; }

long query_tiles(const paged_attn_args& a) {
  const int rows = rows_per_tile(a);
  return static_cast<long>((a.max_qo_len + rows - 1) / rows) * a.num_seqs * a.num_heads;
}

// Key splits for tables of up to `pages` pages per sequence.  The split count
// s (at most 64, and at least two pages per split so the merge traffic stays
// small against the K/V reads) minimises the modelled time: rounds of
// workgroups, ceil(tiles * s / slots), times the work of one workgroup, pages /
// s plus a fixed 3/4 page (prologue, first loads, epilogue), plus the split
// partials' round trip and merge when s > 1 (about 1/320 of a page-round per
// query tile and split: 70 KB of fp16 partials per 256-row tile written and
// read back at HBM rate, against one page of a 256-row tile's products).
// A LingBot frame's 16 tiles get 16 splits (one round); 6 batched streams' 96
// tiles get 8 (three full rounds) rather than 3 (a full round and a nearly
// empty one); a 10,992-query chunk's 352 tiles of 512 rows over 172 pages get
// 5 (seven rounds, the last 88% full) rather than 1 (two rounds, the second
// 38% full); the 137,400-query global call's 4,304 tiles stay unsplit.
// A split is taken only when it beats one split by 3% in the model.
int splits_for_pages(const paged_attn_args& a, long tiles, int pages) {
  const long slots = workgroup_slots(a);
  if (pages <= 1) return 1;
  const int smax = std::max(1, std::min(64, pages / 2));
  auto cost = [&](int s) {
    const long rounds = (tiles * s + slots - 1) / slots;
    const double merge = s > 1 ? static_cast<double>(tiles) * s / 320.0 : 0.0;
    return static_cast<double>(rounds) * (static_cast<double>(pages) / s + 0.75) + merge;
  };
  double best = 0.0;
  int bs = 1;
  for (int s = 2; s <= smax; ++s) {
    const double c = cost(s);
    if (bs == 1 || c < best * (1.0 - 1e-9)) {
      best = c;
      bs = s;
    }
  }
  // Split only for a clear modelled gain (3%): the model is coarse, and a
  // split adds partial traffic that a near tie does not repay.
  return bs > 1 && best < 0.97 * cost(1) ? bs : 1;
}

int choose_splits(const paged_attn_args& a) {
  if (a.num_splits > 0) return std::max(1, std::min(a.num_splits, std::max(1, a.max_kv_pages)));
  return splits_for_pages(a, query_tiles(a), a.max_kv_pages);
}

// The largest split count any call with up to a.max_kv_pages pages per
// sequence (and otherwise these arguments) can get: workspace sizes use it, so
// a workspace sized for a cache's largest table serves every smaller one.
int max_splits(const paged_attn_args& a) {
  if (a.num_splits > 0) return choose_splits(a);
  const long tiles = query_tiles(a);
  int m = 1;
  for (int w = 1; w <= a.max_kv_pages; ++w) m = std::max(m, splits_for_pages(a, tiles, w));
  return m;
}

int check_attn_args(const paged_attn_args* a) {
  if (!a) return fail(KVC_ERR_INVALID_ARGUMENT, "args is NULL");
  if (a->dtype != KVC_DTYPE_BF16 && a->dtype != KVC_DTYPE_F32 && a->dtype != KVC_DTYPE_FP8_E4M3)
    return fail(KVC_ERR_INVALID_ARGUMENT, "bad dtype %d", a->dtype);
  if (a->head_dim != kvc::kHeadDim) return fail(KVC_ERR_UNSUPPORTED, "head_dim %d (kernels need 64)", a->head_dim);
  if (a->page_size <= 0 || a->page_size % kvc::kKeyTile != 0)
    return fail(KVC_ERR_UNSUPPORTED, "page_size %d (kernels need a multiple of 64)", a->page_size);
  if (a->num_heads <= 0 || a->num_seqs < 0 || a->total_q < 0 || a->max_qo_len < 0 || a->max_kv_pages < 0 ||
      a->num_pool_pages < 0 || a->num_splits < 0)
    return fail(KVC_ERR_INVALID_ARGUMENT, "negative size in paged_attn_args");
  if (!(std::isfinite(a->sm_scale) && a->sm_scale > 0.f))
    return fail(KVC_ERR_INVALID_ARGUMENT, "sm_scale must be finite and > 0");
  // the kernels move q, the pools, o and the split partials in 16-byte accesses
  const uintptr_t ptrs = reinterpret_cast<uintptr_t>(a->q) | reinterpret_cast<uintptr_t>(a->k_pool) |
                         reinterpret_cast<uintptr_t>(a->v_pool) | reinterpret_cast<uintptr_t>(a->o) |
                         reinterpret_cast<uintptr_t>(a->workspace);
  if (ptrs & 15) return fail(KVC_ERR_INVALID_ARGUMENT, "q, k_pool, v_pool, o and workspace must be 16-byte aligned");
  return KVC_OK;
}

size_t workspace_for(const paged_attn_args& a, int splits) {
  if (splits <= 1) return 0;
  const size_t rh = static_cast<size_t>(a.total_q) * a.num_heads;
  const size_t o = static_cast<size_t>(splits) * rh * kvc::kHeadDim * sizeof(float);
  const size_t l = static_cast<size_t>(splits) * rh * sizeof(float);
  return ((o + 255) & ~size_t(255)) + l;
}

// Fills the kernel parameters shared by both table sources; returns the
// split count through *splits_out.
int setup_attn(const paged_attn_args& a, kvc::AttnParams& p, int* splits_out) {
  const int splits = choose_splits(a);
  const size_t need = workspace_for(a, splits);
  if (need > 0 && (!a.workspace || a.workspace_bytes < need))
    return fail(KVC_ERR_BUFFER_TOO_SMALL, "workspace needs %zu bytes", need);
  const int rows = rows_per_tile(a);
  const long q_tiles = (a.max_qo_len + rows - 1) / rows;
  const long groups = static_cast<long>(a.num_seqs) * a.num_heads * splits;
  const long groups_padded = (groups + kXcds - 1) / kXcds * kXcds;
  if (q_tiles * groups_padded > 0x7fffffffL) return fail(KVC_ERR_UNSUPPORTED, "grid too large");
  p = kvc::AttnParams{};
  p.q = a.q;
  p.k_pool = a.k_pool;
  p.v_pool = a.v_pool;
  p.o = a.o;
  p.lse = a.lse;
  if (splits > 1) {
    const size_t rh = static_cast<size_t>(a.total_q) * a.num_heads;
    p.part_o = static_cast<float*>(a.workspace);
    const size_t obytes = (static_cast<size_t>(splits) * rh * kvc::kHeadDim * sizeof(float) + 255) & ~size_t(255);
    p.part_lse = reinterpret_cast<float*>(static_cast<char*>(a.workspace) + obytes);
    // The fp16 form of the bf16/FP8 kernels uses the first half of the O
    // region for the values and the second half for the scales.
    p.part_o16 = static_cast<_Float16*>(a.workspace);
    p.part_scale = reinterpret_cast<float*>(static_cast<char*>(a.workspace) + obytes / 2);
  }
  p.qo_indptr = a.qo_indptr;
  p.kv_indptr = a.kv_indptr;
  p.page_ids = a.page_ids;
  p.page_lens = a.page_lens;
  p.num_heads = a.num_heads;
  p.page_size = a.page_size;
  p.num_pool_pages = a.num_pool_pages;
  p.num_seqs = a.num_seqs;
  p.total_q = a.total_q;
  p.q_tiles = static_cast<int32_t>(q_tiles);
  p.num_splits = splits;
  p.groups = static_cast<int32_t>(groups);
  p.groups_padded = static_cast<int32_t>(groups_padded);
  p.sm_scale = a.sm_scale;
  p.scale_log2 = a.sm_scale * 1.4426950408889634f;
  *splits_out = splits;
  return KVC_OK;
}

template <class Src>
int launch_attn(const paged_attn_args& a, const Src& src, int splits, hipStream_t st) {
  const kvc::AttnParams& p = kvc::attn_base(src);
  if (kvc::g_kernel_start) {
    const hipError_t e = hipEventRecord(kvc::g_kernel_start, st);
    if (e != hipSuccess) return fail(KVC_ERR_DEVICE, "recording the kernel-start event: %s", hipGetErrorString(e));
  }
  hipError_t e = a.dtype == KVC_DTYPE_BF16        ? kvc::launch_attn_bf16(src, choose_waves(a), st)
                 : a.dtype == KVC_DTYPE_FP8_E4M3 ? kvc::launch_attn_fp8kv(src, choose_waves(a), st)
                                                 : kvc::launch_attn_f32(src, st);
  if (e != hipSuccess) return fail(KVC_ERR_DEVICE, "attention launch: %s", hipGetErrorString(e));
  if (kvc::g_kernel_done) {
    e = hipEventRecord(kvc::g_kernel_done, st);
    if (e != hipSuccess) return fail(KVC_ERR_DEVICE, "recording the kernel-done event: %s", hipGetErrorString(e));
  }
  if (splits > 1) {
    // fp32 caches: fp32 partials; bf16 and FP8 caches: fp16 partials, o bf16
    e = a.dtype == KVC_DTYPE_F32
            ? kvc::launch_attn_merge(KVC_DTYPE_F32, splits, a.total_q, a.num_heads, p.part_o, p.part_lse, a.o,
                                     a.lse, st)
            : kvc::launch_attn_merge16(splits, a.total_q, a.num_heads, p.part_o16, p.part_scale, p.part_lse, a.o,
                                       a.lse, st);
    if (e != hipSuccess) return fail(KVC_ERR_DEVICE, "merge launch: %s", hipGetErrorString(e));
  }
  return KVC_OK;
}

// Attention arguments of one cache-level step (single sequence).
paged_attn_args cache_attn_args(const kvc_t* c, int32_t num_q, int32_t num_entries, float sm_scale) {
  const kvc_config& cfg = c->pc.config();
  paged_attn_args a{};
  a.dtype = cfg.dtype;
  a.num_heads = cfg.num_heads;
  a.head_dim = cfg.head_dim;
  a.page_size = cfg.page_size;
  a.sm_scale = sm_scale > 0.f ? sm_scale : 1.f / std::sqrt(static_cast<float>(cfg.head_dim));
  a.num_seqs = 1;
  a.total_q = num_q;
  a.max_qo_len = num_q;
  a.max_kv_pages = num_entries;
  a.num_pool_pages = c->pc.num_pages();
  a.num_splits = 0;
  a.k_pool = c->k_pool;
  a.v_pool = c->v_pool;
  return a;
}

// Whether a table of n entries of cache c can travel in the launch arguments.
bool inline_table_ok(const kvc_t* c, int32_t n) {
  return n <= kvc::kMaxInlinePages && c->pc.num_pages() <= kvc::kInlineMaxPid + 1 &&
         c->pc.config().page_size <= 4095;
}

// Workspace bytes at its start that hold a device copy of a table of n
// entries: ids, lens, then the query and entry index pairs of one sequence.
size_t table_region_bytes(int32_t n) { return (static_cast<size_t>(2 * n + 4) * sizeof(int32_t) + 255) & ~size_t(255); }

// Launch over a table that travels in the launch arguments (n <=
// kMaxInlinePages entries; a.q, a.o, a.lse, a.workspace set).
int launch_inline(paged_attn_args& a, const int32_t* ids, const int32_t* lens, int32_t n, hipStream_t st) {
  if (int s = check_attn_args(&a)) return s;
  static thread_local kvc::AttnParamsInline pi;
  int splits = 1;
  if (int s = setup_attn(a, pi.base, &splits)) return s;
  pi.num_entries = n;
  pi.qo[0] = 0;
  pi.qo[1] = a.total_q;
  pi.kv[0] = 0;
  pi.kv[1] = n;
  for (int32_t i = 0; i < n; ++i)
    pi.entries[i] = static_cast<uint32_t>(ids[i]) | (static_cast<uint32_t>(lens[i]) << kvc::kInlinePidBits);
  return launch_attn(a, pi, splits, st);
}

// Attention of one cache's queries over an explicit table (ids, lens; n
// entries of this cache's pool).  Tables of up to 640 entries travel in the
// launch arguments; longer ones are staged in pinned host memory and copied
// asynchronously to the start of the workspace on `stream`.
int attend_table(const kvc_t* c, const int32_t* ids, const int32_t* lens, int32_t n, const void* q, int32_t num_q,
                 float sm_scale, void* o, float* lse, void* workspace, size_t workspace_bytes, kvc_stream_t stream) {
  if (!c->k_pool) return fail(KVC_ERR_INVALID_ARGUMENT, "host-only cache has no device pools");
  if (num_q < 0 || !(sm_scale >= 0.f) || !std::isfinite(sm_scale))
    return fail(KVC_ERR_INVALID_ARGUMENT, "bad num_q or sm_scale");
  if (num_q == 0) return KVC_OK;
  if (!q || !o) return fail(KVC_ERR_INVALID_ARGUMENT, "NULL q or o");
  paged_attn_args a = cache_attn_args(c, num_q, n, sm_scale);
  a.q = q;
  a.o = o;
  a.lse = lse;
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (inline_table_ok(c, n)) {
    a.workspace = workspace;
    a.workspace_bytes = workspace_bytes;
    return launch_inline(a, ids, lens, n, st);
  }
  // device table at the start of the workspace, split partials after it
  const size_t tb = table_region_bytes(n);
  if (!workspace || workspace_bytes < tb)
    return fail(KVC_ERR_BUFFER_TOO_SMALL, "a table of %d entries needs a workspace of at least %zu bytes", n, tb);
  a.workspace = static_cast<char*>(workspace) + tb;
  a.workspace_bytes = workspace_bytes - tb;
  if (int s = check_attn_args(&a)) return s;
  kvc::AttnParams p;
  int splits = 1;
  if (int s = setup_attn(a, p, &splits)) return s;
  const size_t words = static_cast<size_t>(2 * n + 4);
  int slot = 0;
  int32_t* h = c->ring.acquire(words, &slot);
  if (!h) return KVC_ERR_DEVICE;
  std::copy(ids, ids + n, h);
  std::copy(lens, lens + n, h + n);
  h[2 * n] = 0;
  h[2 * n + 1] = num_q;
  h[2 * n + 2] = 0;
  h[2 * n + 3] = n;
  int32_t* d = static_cast<int32_t*>(workspace);
  hipError_t e = hipMemcpyAsync(d, h, words * sizeof(int32_t), hipMemcpyHostToDevice, st);
  if (e != hipSuccess) return fail(KVC_ERR_DEVICE, "table upload: %s", hipGetErrorString(e));
  e = hipEventRecord(c->ring.done[slot], st);
  if (e != hipSuccess) {
    // the copy is queued but cannot be tracked: let it finish before the slot
    // can be written again
    (void)hipStreamSynchronize(st);
    return fail(KVC_ERR_DEVICE, "table upload: %s", hipGetErrorString(e));
  }
  c->ring.in_flight[slot] = true;
  p.page_ids = d;
  p.page_lens = d + n;
  p.qo_indptr = d + 2 * n;
  p.kv_indptr = d + 2 * n + 2;
  return launch_attn(a, p, splits, st);
}

// Workspace bytes for any attention call of cache c with num_q queries: the
// split partials of the largest split count its tables can get, plus the
// device-table region when its tables can outgrow the launch arguments.
int cache_workspace_bytes(const kvc_t* c, int32_t num_q, size_t* bytes) {
  const int32_t max_entries = c->pc.num_pages();
  const paged_attn_args a = cache_attn_args(c, num_q, max_entries, 0.f);
  if (int s = check_attn_args(&a)) return s;
  *bytes = workspace_for(a, max_splits(a)) + (inline_table_ok(c, max_entries) ? 0 : table_region_bytes(max_entries));
  return KVC_OK;
}

// Checks a batch of caches for kvc_attend_batch and derives its launch
// arguments: every cache's pool offset (whole pages from the lowest pool
// pointer of the batch, the same for K and V) and the combined sizes.
int batch_args(const kvc_t* const* caches, int32_t n, const int32_t* qo, float sm_scale, paged_attn_args* a,
               int32_t* page_off) {
  if (!caches || n <= 0 || !qo) return fail(KVC_ERR_INVALID_ARGUMENT, "bad batch");
  if (n > kvc::kMaxInlineSeqs) return fail(KVC_ERR_UNSUPPORTED, "batch of %d caches (at most %d)", n, kvc::kMaxInlineSeqs);
  if (!(sm_scale >= 0.f) || !std::isfinite(sm_scale)) return fail(KVC_ERR_INVALID_ARGUMENT, "bad sm_scale");
  if (qo[0] != 0) return fail(KVC_ERR_INVALID_ARGUMENT, "qo_indptr[0] must be 0");
  const kvc_t* c0 = caches[0];
  if (!c0) return fail(KVC_ERR_INVALID_ARGUMENT, "NULL cache in batch");
  const kvc_config& f = c0->pc.config();
  const char* base_k = nullptr;
  const char* base_v = nullptr;
  int32_t entries = 0, max_q = 0;
  for (int32_t i = 0; i < n; ++i) {
    const kvc_t* c = caches[i];
    if (!c) return fail(KVC_ERR_INVALID_ARGUMENT, "NULL cache in batch");
    if (!c->k_pool) return fail(KVC_ERR_INVALID_ARGUMENT, "host-only cache %d has no device pools", i);
    const kvc_config& g = c->pc.config();
    if (g.dtype == KVC_DTYPE_FP8_E4M3)
      return fail(KVC_ERR_UNSUPPORTED, "cache %d: FP8 caches are not batched (their exponents sit at the end of "
                  "each cache's own pool buffer)", i);
    if (g.num_heads != f.num_heads || g.head_dim != f.head_dim || g.page_size != f.page_size || g.dtype != f.dtype)
      return fail(KVC_ERR_INVALID_ARGUMENT, "cache %d: heads, head_dim, page_size and dtype must match the batch", i);
    if (qo[i + 1] < qo[i]) return fail(KVC_ERR_INVALID_ARGUMENT, "qo_indptr must be non-decreasing");
    max_q = std::max(max_q, qo[i + 1] - qo[i]);
    entries += c->pc.visible_count();
    const char* k = static_cast<const char*>(c->k_pool);
    const char* v = static_cast<const char*>(c->v_pool);
    if (!base_k || k < base_k) base_k = k;
    if (!base_v || v < base_v) base_v = v;
  }
  if (entries > kvc::kMaxInlinePages)
    return fail(KVC_ERR_UNSUPPORTED, "batch has %d table entries (at most %d)", entries, kvc::kMaxInlinePages);
  const size_t page_bytes = static_cast<size_t>(f.num_heads) * f.page_size * f.head_dim * elem_size(f.dtype);
  int64_t pool_pages = 0;
  for (int32_t i = 0; i < n; ++i) {
    const size_t dk = static_cast<size_t>(static_cast<const char*>(caches[i]->k_pool) - base_k);
    const size_t dv = static_cast<size_t>(static_cast<const char*>(caches[i]->v_pool) - base_v);
    if (dk % page_bytes != 0 || dk != dv)
      return fail(KVC_ERR_INVALID_ARGUMENT,
                  "cache %d: pools must sit whole pages into one shared K and one shared V allocation, "
                  "at the same page offset", i);
    const int64_t off = static_cast<int64_t>(dk / page_bytes);
    pool_pages = std::max<int64_t>(pool_pages, off + caches[i]->pc.num_pages());
    if (pool_pages > kvc::kInlineMaxPid + 1) return fail(KVC_ERR_UNSUPPORTED, "shared pool too large for inline tables");
    page_off[i] = static_cast<int32_t>(off);
  }
  if (f.page_size > 4095) return fail(KVC_ERR_UNSUPPORTED, "page size too large for inline tables");
  *a = paged_attn_args{};
  a->dtype = f.dtype;
  a->num_heads = f.num_heads;
  a->head_dim = f.head_dim;
  a->page_size = f.page_size;
  a->sm_scale = sm_scale > 0.f ? sm_scale : 1.f / std::sqrt(static_cast<float>(f.head_dim));
  a->num_seqs = n;
  a->total_q = qo[n];
  a->max_qo_len = max_q;
  int32_t max_pages = 0;
  for (int32_t i = 0; i < n; ++i) max_pages = std::max(max_pages, caches[i]->pc.visible_count());
  a->max_kv_pages = max_pages;
  a->num_pool_pages = static_cast<int32_t>(pool_pages);
  a->num_splits = 0;
  a->k_pool = base_k;
  a->v_pool = base_v;
  return KVC_OK;
}

}  // namespace

namespace kvc {

int attend_fixed_workspace(const kvc_t* c, const void* q, int32_t num_q, float sm_scale, void* o, float* lse,
                           void* workspace, size_t workspace_bytes, kvc_stream_t stream) {
  if (!c) return fail(KVC_ERR_INVALID_ARGUMENT, "NULL handle");
  if (!c->k_pool) return fail(KVC_ERR_INVALID_ARGUMENT, "host-only cache has no device pools");
  if (num_q < 0 || !(sm_scale >= 0.f) || !std::isfinite(sm_scale))
    return fail(KVC_ERR_INVALID_ARGUMENT, "bad num_q or sm_scale");
  if (num_q == 0) return KVC_OK;
  if (!q || !o) return fail(KVC_ERR_INVALID_ARGUMENT, "NULL q or o");
  const int32_t n = c->pc.visible_count();
  if (!inline_table_ok(c, n))
    return fail(KVC_ERR_UNSUPPORTED,
                "the visible table has %d entries; without allocation at most %d travel in the launch arguments "
                "(longer tables need staging memory: use kvc_attend)", n, kvc::kMaxInlinePages);
  int32_t ids[kvc::kMaxInlinePages], lens[kvc::kMaxInlinePages];
  c->pc.visible_table(ids, lens);
  paged_attn_args a = cache_attn_args(c, num_q, n, sm_scale);
  a.q = q;
  a.o = o;
  a.lse = lse;
  a.workspace = workspace;
  a.workspace_bytes = workspace_bytes;
  if (int s = check_attn_args(&a)) return s;
  // The split count kvc_attend would take, or the largest whose partials fit.
  int splits = choose_splits(a);
  while (splits > 1 && workspace_for(a, splits) > workspace_bytes) --splits;
  a.num_splits = splits;
  return launch_inline(a, ids, lens, n, reinterpret_cast<hipStream_t>(stream));
}

}  // namespace kvc

extern "C" {

const char* kvc_strerror(int status) {
  switch (status) {
    case KVC_OK: return "ok";
    case KVC_ERR_INVALID_ARGUMENT: return "invalid argument";
    case KVC_ERR_OUT_OF_PAGES: return "out of pages";
    case KVC_ERR_NO_UNDO: return "no append to roll back";
    case KVC_ERR_BUFFER_TOO_SMALL: return "buffer too small";
    case KVC_ERR_UNSUPPORTED: return "unsupported";
    case KVC_ERR_DEVICE: return "device error";
    case KVC_ERR_HOST_MEMORY: return "out of host memory";
    case KVC_ERR_INTERNAL: return "internal error";
    default: return "unknown status";
  }
}

const char* kvc_last_error(void) { return kvc::g_last_error; }

int kvc_version(void) { return 300; }

int kvc_required_pages(const kvc_config* cfg, int32_t* num_pages) {
  return guarded("kvc_required_pages", [&] {
    if (!cfg || !num_pages) return fail(KVC_ERR_INVALID_ARGUMENT, "NULL argument");
    if (int s = kvc::PageCache::validate(*cfg)) return fail(s, "invalid kvc_config");
    const int32_t n = kvc::PageCache::required_pages(*cfg);
    if (n < 0) return fail(KVC_ERR_INVALID_ARGUMENT, "page count overflows int32");
    *num_pages = n;
    return static_cast<int>(KVC_OK);
  });
}

int kvc_pool_bytes(const kvc_config* cfg, size_t* bytes) {
  return guarded("kvc_pool_bytes", [&] {
    if (!cfg || !bytes) return fail(KVC_ERR_INVALID_ARGUMENT, "NULL argument");
    if (int s = kvc::PageCache::validate(*cfg)) return fail(s, "invalid kvc_config");
    const int32_t n = cfg->num_pages > 0 ? cfg->num_pages : kvc::PageCache::required_pages(*cfg);
    if (n < 0) return fail(KVC_ERR_INVALID_ARGUMENT, "page count overflows int32");
    *bytes = pool_bytes(*cfg, n);
    return static_cast<int>(KVC_OK);
  });
}

int kvc_create(const kvc_config* cfg, void* k_pool, void* v_pool, kvc_t** out) {
  return guarded("kvc_create", [&] {
    if (!cfg || !out) return fail(KVC_ERR_INVALID_ARGUMENT, "NULL argument");
    if (int s = kvc::PageCache::validate(*cfg)) return fail(s, "invalid kvc_config");
    if ((k_pool == nullptr) != (v_pool == nullptr))
      return fail(KVC_ERR_INVALID_ARGUMENT, "k_pool and v_pool must both be set or both be NULL");
    if (k_pool && !device_shapes_ok(*cfg))
      return fail(KVC_ERR_UNSUPPORTED, "device pools need head_dim 64 and page_size a multiple of 64");
    const int64_t u = (int64_t(cfg->patch_tokens) + cfg->page_size - 1) / cfg->page_size;
    if (k_pool && u > kvc::kMaxUnitPages)
      return fail(KVC_ERR_UNSUPPORTED, "a unit spans %lld pages (max %d)", static_cast<long long>(u),
                  kvc::kMaxUnitPages);
    if (kvc::PageCache::required_pages(*cfg) < 0 && cfg->num_pages == 0)
      return fail(KVC_ERR_INVALID_ARGUMENT, "page count overflows int32");
    kvc_cache* c = new kvc_cache(*cfg);  // bad_alloc -> KVC_ERR_HOST_MEMORY
    c->k_pool = k_pool;
    c->v_pool = v_pool;
    *out = c;
    return static_cast<int>(KVC_OK);
  });
}

int kvc_destroy(kvc_t* cache) {
  return guarded("kvc_destroy", [&] {
    delete cache;
    return static_cast<int>(KVC_OK);
  });
}

int kvc_append_frame(kvc_t* c, const void* k_unit, const void* v_unit, kvc_stream_t stream) {
  return guarded("kvc_append_frame", [&] { return kvc::append_unit(c, k_unit, v_unit, stream, nullptr, nullptr); });
}

}  // extern "C"

int kvc::append_unit(kvc_t* c, const void* k_unit, const void* v_unit, kvc_stream_t stream, void* k_copy,
                     void* v_copy) {
  if (!c) return fail(KVC_ERR_INVALID_ARGUMENT, "NULL handle");
  const bool device = c->k_pool != nullptr;
  if (device && (!k_unit || !v_unit)) return fail(KVC_ERR_INVALID_ARGUMENT, "device cache needs K and V");
  if (!device && (k_unit || v_unit)) return fail(KVC_ERR_INVALID_ARGUMENT, "host-only cache takes NULL K and V");
  if ((reinterpret_cast<uintptr_t>(k_unit) | reinterpret_cast<uintptr_t>(v_unit)) & 15)
    return fail(KVC_ERR_INVALID_ARGUMENT, "K and V must be 16-byte aligned");
  if (!device) {
    const int s = c->pc.append();
    return s == KVC_OK ? s : fail(s, "append needs %d pages", c->pc.unit_pages());
  }
  // plan, launch, then commit: a failed launch leaves the cache unchanged
  kvc::AppendPlan plan;
  kvc::AppendParams p{};
  if (int s = c->pc.plan(&plan, p.unit_pages)) return fail(s, "append needs %d pages", c->pc.unit_pages());
  const kvc_config& cfg = c->pc.config();
  p.k_src = k_unit;
  p.v_src = v_unit;
  p.k_pool = c->k_pool;
  p.v_pool = c->v_pool;
  p.num_heads = cfg.num_heads;
  p.page_size = cfg.page_size;
  p.patch_tokens = cfg.patch_tokens;
  p.special_tokens = cfg.special_tokens;
  p.special_page0 = plan.special_page0;
  p.special_slot0 = plan.special_slot0;
  p.special_count0 = plan.special_count0;
  p.special_page1 = plan.special_page1;
  p.num_unit_pages = plan.num_unit_pages;
  p.k_copy = k_copy;
  p.v_copy = v_copy;
  if (cfg.dtype == KVC_DTYPE_FP8_E4M3) {
    // row exponents follow the codes in each pool buffer
    const size_t codes = static_cast<size_t>(c->pc.num_pages()) * cfg.num_heads * cfg.page_size * cfg.head_dim;
    p.k_exp = static_cast<char*>(c->k_pool) + codes;
    p.v_exp = static_cast<char*>(c->v_pool) + codes;
  }
  const hipError_t e = kvc::launch_kv_append(p, cfg.dtype, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(KVC_ERR_DEVICE, "append launch: %s", hipGetErrorString(e));
  c->pc.commit();
  return static_cast<int>(KVC_OK);
}

extern "C" {

int kvc_rollback_last_frame(kvc_t* c) {
  return guarded("kvc_rollback_last_frame", [&] {
    if (!c) return fail(KVC_ERR_INVALID_ARGUMENT, "NULL handle");
    const int s = c->pc.rollback();
    return s == KVC_OK ? s : fail(s, "nothing to roll back");
  });
}

int kvc_reset(kvc_t* c) {
  return guarded("kvc_reset", [&] {
    if (!c) return fail(KVC_ERR_INVALID_ARGUMENT, "NULL handle");
    c->pc.reset();
    return static_cast<int>(KVC_OK);
  });
}

int kvc_build_visible_table(const kvc_t* c, int32_t* page_ids, int32_t* page_lens, int32_t capacity,
                            int32_t* num_pages, int32_t* last_page_len) {
  return guarded("kvc_build_visible_table", [&] {
    if (!c || !num_pages) return fail(KVC_ERR_INVALID_ARGUMENT, "NULL argument");
    const int32_t n = c->pc.visible_count();
    *num_pages = n;
    if ((page_ids || page_lens) && capacity < n)
      return fail(KVC_ERR_BUFFER_TOO_SMALL, "table needs %d entries, capacity %d", n, capacity);
    if (page_ids || page_lens) c->pc.visible_table(page_ids, page_lens);
    if (last_page_len) {
      // the last entry's length, read without a caller array when none was given
      if (page_lens) {
        *last_page_len = n ? page_lens[n - 1] : 0;
      } else {
        std::vector<int32_t> lens(static_cast<size_t>(n));
        c->pc.visible_table(nullptr, lens.data());
        *last_page_len = n ? lens[n - 1] : 0;
      }
    }
    return static_cast<int>(KVC_OK);
  });
}

int kvc_get_state(const kvc_t* c, kvc_state* st) {
  return guarded("kvc_get_state", [&] {
    if (!c || !st) return fail(KVC_ERR_INVALID_ARGUMENT, "NULL argument");
    if (st->capacity < c->pc.num_pages() &&
        (st->free_pages || st->scale_pages || st->window_pages || st->special_pages))
      return fail(KVC_ERR_BUFFER_TOO_SMALL, "state arrays need %d entries", c->pc.num_pages());
    c->pc.state(st);
    return static_cast<int>(KVC_OK);
  });
}

int paged_attn_workspace_size(const paged_attn_args* a, size_t* bytes) {
  return guarded("paged_attn_workspace_size", [&] {
    if (!bytes) return fail(KVC_ERR_INVALID_ARGUMENT, "NULL bytes");
    if (int s = check_attn_args(a)) return s;
    *bytes = workspace_for(*a, max_splits(*a));
    return static_cast<int>(KVC_OK);
  });
}

int paged_attn_num_splits(const paged_attn_args* a, int32_t* num_splits) {
  return guarded("paged_attn_num_splits", [&] {
    if (!num_splits) return fail(KVC_ERR_INVALID_ARGUMENT, "NULL num_splits");
    if (int s = check_attn_args(a)) return s;
    *num_splits = choose_splits(*a);
    return static_cast<int>(KVC_OK);
  });
}

int paged_attn_fwd(const paged_attn_args* a, kvc_stream_t stream) {
  return guarded("paged_attn_fwd", [&] {
    if (int s = check_attn_args(a)) return s;
    if (a->num_seqs == 0 || a->total_q == 0 || a->max_qo_len == 0) return static_cast<int>(KVC_OK);
    if (!a->qo_indptr || !a->kv_indptr || !a->q || !a->o)
      return fail(KVC_ERR_INVALID_ARGUMENT, "NULL device pointer");
    if (a->max_kv_pages > 0 && (!a->page_ids || !a->page_lens || !a->k_pool || !a->v_pool))
      return fail(KVC_ERR_INVALID_ARGUMENT, "NULL table or pool pointer");
    kvc::AttnParams p;
    int splits = 1;
    if (int s = setup_attn(*a, p, &splits)) return s;
    return launch_attn(*a, p, splits, reinterpret_cast<hipStream_t>(stream));
  });
}

int kvc_attend_workspace_size(const kvc_t* c, int32_t num_q, size_t* bytes) {
  return guarded("kvc_attend_workspace_size", [&] {
    if (!c || !bytes || num_q < 0) return fail(KVC_ERR_INVALID_ARGUMENT, "bad argument");
    return cache_workspace_bytes(c, num_q, bytes);
  });
}

int kvc_attend(const kvc_t* c, const void* q, int32_t num_q, float sm_scale, void* o, float* lse,
               void* workspace, size_t workspace_bytes, kvc_stream_t stream) {
  return guarded("kvc_attend", [&] {
    if (!c) return fail(KVC_ERR_INVALID_ARGUMENT, "NULL handle");
    const int32_t n = c->pc.visible_count();
    if (n <= kvc::kMaxInlinePages) {
      int32_t ids[kvc::kMaxInlinePages], lens[kvc::kMaxInlinePages];
      c->pc.visible_table(ids, lens);
      return attend_table(c, ids, lens, n, q, num_q, sm_scale, o, lse, workspace, workspace_bytes, stream);
    }
    std::vector<int32_t> ids(static_cast<size_t>(n)), lens(static_cast<size_t>(n));
    c->pc.visible_table(ids.data(), lens.data());
    return attend_table(c, ids.data(), lens.data(), n, q, num_q, sm_scale, o, lse, workspace, workspace_bytes,
                        stream);
  });
}

int kvc_build_subset_table(const kvc_t* c, float keep_ratio, uint64_t seed, int32_t keep_first, int32_t keep_last,
                           int32_t* page_ids, int32_t* page_lens, int32_t capacity, int32_t* num_pages) {
  return guarded("kvc_build_subset_table", [&] {
    if (!c || !num_pages) return fail(KVC_ERR_INVALID_ARGUMENT, "NULL argument");
    if (!(keep_ratio > 0.f && keep_ratio <= 1.f)) return fail(KVC_ERR_INVALID_ARGUMENT, "keep_ratio must be in (0, 1]");
    if (keep_first < 0 || keep_last < 0) return fail(KVC_ERR_INVALID_ARGUMENT, "negative keep_first/keep_last");
    const int32_t n = c->pc.visible_count();
    std::vector<int32_t> ids(static_cast<size_t>(n)), lens(static_cast<size_t>(n));
    c->pc.visible_table(ids.data(), lens.data());
    std::vector<int32_t> sid(static_cast<size_t>(n)), slen(static_cast<size_t>(n));
    const int32_t m = kvc::subset_select(ids.data(), lens.data(), n, keep_ratio, seed, keep_first, keep_last,
                                         sid.data(), slen.data());
    *num_pages = m;
    if (capacity < m || (m > 0 && (!page_ids || !page_lens)))
      return fail(KVC_ERR_BUFFER_TOO_SMALL, "subset table needs %d entries", m);
    std::copy(sid.begin(), sid.begin() + m, page_ids);
    std::copy(slen.begin(), slen.begin() + m, page_lens);
    return static_cast<int>(KVC_OK);
  });
}

int kvc_attend_subset(const kvc_t* c, float keep_ratio, uint64_t seed, int32_t keep_first, int32_t keep_last,
                      const void* q, int32_t num_q, float sm_scale, void* o, float* lse, void* workspace,
                      size_t workspace_bytes, kvc_stream_t stream) {
  return guarded("kvc_attend_subset", [&] {
    if (!c) return fail(KVC_ERR_INVALID_ARGUMENT, "NULL handle");
    if (!(keep_ratio > 0.f && keep_ratio <= 1.f)) return fail(KVC_ERR_INVALID_ARGUMENT, "keep_ratio must be in (0, 1]");
    if (keep_first < 0 || keep_last < 0) return fail(KVC_ERR_INVALID_ARGUMENT, "negative keep_first/keep_last");
    const int32_t n = c->pc.visible_count();
    std::vector<int32_t> ids(static_cast<size_t>(n)), lens(static_cast<size_t>(n));
    c->pc.visible_table(ids.data(), lens.data());
    std::vector<int32_t> sid(static_cast<size_t>(n)), slen(static_cast<size_t>(n));
    const int32_t m = kvc::subset_select(ids.data(), lens.data(), n, keep_ratio, seed, keep_first, keep_last,
                                         sid.data(), slen.data());
    return attend_table(c, sid.data(), slen.data(), m, q, num_q, sm_scale, o, lse, workspace, workspace_bytes,
                        stream);
  });
}

int kvc_attend_batch_workspace_size(const kvc_t* const* caches, int32_t num_caches, const int32_t* qo_indptr,
                                    size_t* bytes) {
  return guarded("kvc_attend_batch_workspace_size", [&] {
    if (!bytes) return fail(KVC_ERR_INVALID_ARGUMENT, "NULL bytes");
    paged_attn_args a;
    int32_t off[kvc::kMaxInlineSeqs];
    if (int s = batch_args(caches, num_caches, qo_indptr, 0.f, &a, off)) return s;
    if (int s = check_attn_args(&a)) return s;
    *bytes = workspace_for(a, max_splits(a));
    return static_cast<int>(KVC_OK);
  });
}

int kvc_attend_batch(const kvc_t* const* caches, int32_t num_caches, const void* q, const int32_t* qo_indptr,
                     float sm_scale, void* o, float* lse, void* workspace, size_t workspace_bytes,
                     kvc_stream_t stream) {
  return guarded("kvc_attend_batch", [&] {
    paged_attn_args a;
    int32_t off[kvc::kMaxInlineSeqs];
    if (int s = batch_args(caches, num_caches, qo_indptr, sm_scale, &a, off)) return s;
    if (a.total_q == 0) return static_cast<int>(KVC_OK);
    if (!q || !o) return fail(KVC_ERR_INVALID_ARGUMENT, "NULL q or o");
    a.q = q;
    a.o = o;
    a.lse = lse;
    a.workspace = workspace;
    a.workspace_bytes = workspace_bytes;
    if (int s = check_attn_args(&a)) return s;
    static thread_local kvc::AttnParamsInline pi;
    int splits = 1;
    if (int s = setup_attn(a, pi.base, &splits)) return s;
    int32_t ids[kvc::kMaxInlinePages], lens[kvc::kMaxInlinePages];
    int32_t e = 0;
    pi.qo[0] = 0;
    pi.kv[0] = 0;
    for (int32_t i = 0; i < num_caches; ++i) {
      const int32_t m = caches[i]->pc.visible_count();
      caches[i]->pc.visible_table(ids + e, lens + e);
      for (int32_t j = e; j < e + m; ++j)
        pi.entries[j] =
            static_cast<uint32_t>(ids[j] + off[i]) | (static_cast<uint32_t>(lens[j]) << kvc::kInlinePidBits);
      e += m;
      pi.qo[i + 1] = qo_indptr[i + 1];
      pi.kv[i + 1] = e;
    }
    pi.num_entries = e;
    return launch_attn(a, pi, splits, reinterpret_cast<hipStream_t>(stream));
  });
}

int paged_attn_merge(int32_t dtype, int32_t num_parts, int32_t rows, int32_t num_heads, int32_t head_dim,
                     const float* partial_o, const float* partial_lse, void* o, float* lse, kvc_stream_t stream) {
  return guarded("paged_attn_merge", [&] {
    if (dtype != KVC_DTYPE_BF16 && dtype != KVC_DTYPE_F32) return fail(KVC_ERR_INVALID_ARGUMENT, "bad dtype");
    if (head_dim != kvc::kHeadDim) return fail(KVC_ERR_UNSUPPORTED, "head_dim %d (need 64)", head_dim);
    if (num_parts <= 0 || rows < 0 || num_heads <= 0) return fail(KVC_ERR_INVALID_ARGUMENT, "bad sizes");
    if (rows == 0) return static_cast<int>(KVC_OK);
    if (!partial_o || !partial_lse || !o) return fail(KVC_ERR_INVALID_ARGUMENT, "NULL pointer");
    // the merge reads partial O and writes O in 16- and 8-byte vectors
    if ((reinterpret_cast<uintptr_t>(partial_o) & 15) || (reinterpret_cast<uintptr_t>(o) & 15))
      return fail(KVC_ERR_INVALID_ARGUMENT, "partial_o and o must be 16-byte aligned");
    const hipError_t e = kvc::launch_attn_merge(dtype, num_parts, rows, num_heads, partial_o, partial_lse, o, lse,
                                                reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(KVC_ERR_DEVICE, "merge launch: %s", hipGetErrorString(e));
    return static_cast<int>(KVC_OK);
  });
}

int kvc_set_kernel_events(void* start, void* done) {
  kvc::g_kernel_start = static_cast<hipEvent_t>(start);
  kvc::g_kernel_done = static_cast<hipEvent_t>(done);
  return KVC_OK;
}

}  // extern "C"
