/*
 * kvc.h - paged sliding-window KV cache and paged attention for MI355X (gfx950).
 *
 * C ABI of libkvc.so.  Plain pointers and sizes only; no C++ or framework
 * types cross this boundary.
 *
 * What the library computes
 *   A per-layer KV cache cut into fixed-size pages that are kept in three
 *   streams ("LingBot-Map Paged KV Cache", section 2): scale pages that are
 *   never evicted, sliding-window patch pages that return to a free list once
 *   outside the window and are reused by the next unit, and append-only
 *   special pages packing the special tokens of many frames (42 frames of 6
 *   tokens per 256-slot page).  The visible page table lists scale, then
 *   window, then special pages; each page carries its valid length, so the
 *   partly filled last page needs no mask.  A non-keyframe is appended,
 *   attended and rolled back (section 3).  The same cache runs the chunked
 *   form of "vLLM-Omni RFC #2727: Reconstruction Engine" (section 1 and 2.3):
 *   a unit is a chunk of frames, the window holds the most recent
 *   sliding_window_num chunks including the current one; an unbounded window
 *   is full global attention and a window of 1 gives independent chunks.
 *   paged_attn_fwd computes softmax attention of query tokens against the
 *   tokens of a page table (no mask), with an online softmax over pages.
 *
 * Allocation policy (fixed so that tables are reproducible):
 *   - free list is a LIFO stack; a fresh cache pops pages 0, 1, 2, ...
 *   - an append pops the unit's patch pages, then (when needed) one special
 *     page; after the pops, the oldest window unit is evicted if the window
 *     holds more than window_units units; evicted pages are pushed in
 *     reverse, so a later pop returns the unit's first page first.
 *   - the first num_scale_units units go to the scale stream, later ones to
 *     the window; every unit's special tokens go to the special stream.
 *   - rollback undoes the last append exactly (single level).
 *
 * Device memory
 *   The caller owns all device memory (pools, Q/K/V/O, tables, workspace).
 *   The library owns host metadata only and allocates no device memory.
 *   Pool layout for a cache with H heads, head_dim d, page size P:
 *     K pool: [num_pages][H][P][d]   (slot-major rows of d elements)
 *     V pool: [num_pages][H][d][P]   (transposed: one row of P slots per dim)
 *   Inside a V row, every group of 16 slots is stored with its middle two
 *   4-slot groups swapped: slot s is at element
 *     (s & ~15) | (s & 3) | ((s & 4) << 1) | ((s & 8) >> 1)
 *   (a self-inverse map).  This is the operand order of the attention
 *   kernel's P*V product, so V tiles go from HBM to LDS unchanged.
 *   Element type is bf16 (2 bytes) or fp32 (4 bytes), per kvc_config.dtype.
 *   K/V/Q/O activations are [tokens][H][d], tokens in order.
 *
 *   FP8 caches (KVC_DTYPE_FP8_E4M3; "vLLM-Omni RFC #2727", section 3.4,
 *   item 5: KV cache FP8 for about half the memory) store K and V both
 *   slot-major, [num_pages][H][P][d] bytes of OCP E4M3 codes, followed in the
 *   same buffer by [num_pages][H][P] int8 row exponents e.  Row (page, head,
 *   slot) holds the token's d values as code * 2^e, e being the smallest
 *   integer in [-127, 127] with max|x| <= 448 * 2^e, each value rounded to
 *   the nearest E4M3 value (ties to even).  Appends take bf16 K/V and quantise
 *   them; attention takes bf16 q and writes bf16 o.
 *
 * Streams and threads
 *   Device work is enqueued on the hipStream_t passed in (0 = null stream)
 *   and is asynchronous to the host.  A handle is not thread-safe; use one
 *   stream for every call on a handle, so that an append that recycles a page
 *   is ordered after earlier attention reads of it.
 *
 * Errors
 *   Every call returns KVC_OK (0) or a negative kvc_status.  On error the
 *   handle's state is unchanged (the one exception, a windowed restart that
 *   fails on the device, is stated at kvc_windowed_append).  No C++ exception
 *   leaves the library: host allocation failures give KVC_ERR_HOST_MEMORY.
 *   kvc_last_error() gives a thread-local message for the last failing call
 *   on the calling thread.
 *
 * Passages cited below
 *   "LingBot-Map Paged KV Cache" (a Chinese-language article; section n is
 *   its n-th numbered section, section 0 its lead paragraph) and "vLLM-Omni
 *   RFC #2727: Reconstruction Engine" (RFC #2727, sections 1-3).
 */
#ifndef KVC_H_
#define KVC_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* kvc_stream_t; /* same type as hipStream_t */

typedef enum kvc_status {
  KVC_OK = 0,
  KVC_ERR_INVALID_ARGUMENT = -1,
  KVC_ERR_OUT_OF_PAGES = -2,
  KVC_ERR_NO_UNDO = -3,
  KVC_ERR_BUFFER_TOO_SMALL = -4,
  KVC_ERR_UNSUPPORTED = -5,
  KVC_ERR_DEVICE = -6,
  KVC_ERR_HOST_MEMORY = -7, /* a host allocation failed */
  KVC_ERR_INTERNAL = -8,    /* an unexpected internal error (a bug) */
} kvc_status;

typedef enum kvc_dtype { KVC_DTYPE_BF16 = 0, KVC_DTYPE_F32 = 1, KVC_DTYPE_FP8_E4M3 = 2 } kvc_dtype;

typedef enum kvc_special_packing {
  /* floor(P / special_tokens) whole frames per special page (42 for 6 tokens
   * in 256 slots); a frame never straddles two pages. */
  KVC_SPECIAL_FRAME_ALIGNED = 0,
  /* special tokens packed back to back; a frame may straddle two pages. */
  KVC_SPECIAL_CONTIGUOUS = 1,
} kvc_special_packing;

typedef struct kvc_config {
  int32_t num_heads;        /* H >= 1 */
  int32_t head_dim;         /* d; device paths need 64 */
  int32_t page_size;        /* P tokens per page; device paths need a multiple of 64 */
  int32_t dtype;            /* kvc_dtype */
  int32_t patch_tokens;     /* tokens per unit in the patch stream (frame 256, VGGT frame 1374, chunk 8*1374) */
  int32_t special_tokens;   /* special tokens per unit, 0 <= X <= P (6 for LingBot-Map frames) */
  int32_t num_scale_units;  /* S: first S units are never evicted */
  int32_t window_units;     /* W: window size in units including the newest; <= 0 = unbounded */
  int32_t special_packing;  /* kvc_special_packing */
  int32_t max_units;        /* most units ever cached at once (sizes the special stream) */
  int32_t num_pages;        /* pool capacity in pages; 0 = kvc_required_pages */
} kvc_config;

/* Snapshot of the host metadata.  The caller provides the arrays, each with
 * room for `capacity` entries (num_pages is always enough).  Page lists are
 * in table order; free_pages runs from the bottom of the stack to the top
 * (the next page popped is free_pages[num_free - 1]). */
typedef struct kvc_state {
  int32_t capacity;
  int32_t* free_pages;
  int32_t* scale_pages;
  int32_t* window_pages;
  int32_t* special_pages;
  int32_t num_free;
  int32_t num_scale_pages;
  int32_t num_window_pages;
  int32_t num_window_units;
  int32_t num_special_pages;
  int32_t special_fill;     /* frames (frame-aligned) or tokens (contiguous) in the last special page */
  int32_t num_units;        /* units currently cached */
  int32_t has_undo;         /* 1 if kvc_rollback_last_frame would succeed */
  int32_t num_pages;        /* pool capacity */
} kvc_state;

typedef struct kvc_cache kvc_t;

/* Pages a cache with this config needs ("LingBot-Map Paged KV Cache",
 * section 0: cache memory stays constant over 10,000+ frames; section 2: the
 * patch cache holds the scale and window frames' pages, each frame's 256
 * patch tokens fill one page, and special pages pack 42 frames each): with a
 * bounded window, min(max_units, S + W + 1) units of ceil(patch_tokens / P)
 * pages (one unit more than the window holds, since an append pops before it
 * evicts), plus the special pages of max_units units; with an unbounded
 * window (RFC #2727, section 2.3: an infinite window is full global
 * attention), max_units units.  *num_pages receives the count.
 * KVC_ERR_INVALID_ARGUMENT for an invalid config or a count past int32. */
int kvc_required_pages(const kvc_config* cfg, int32_t* num_pages);

/* Bytes of one pool (K or V) for cfg (num_pages, or kvc_required_pages when
 * 0): num_pages * H * P * d * sizeof(element); for FP8 caches
 * num_pages * H * P * (d + 1) (codes and row exponents).  The caller
 * allocates the pools once at this size; nothing grows afterwards
 * ("LingBot-Map Paged KV Cache", section 0: constant cache memory). */
int kvc_pool_bytes(const kvc_config* cfg, size_t* bytes);

/* Create a cache: one layer's page pool, free list and three page streams
 * ("LingBot-Map Paged KV Cache", section 2: each layer's KV is cut into
 * fixed-size pages; a fresh free list pops pages 0, 1, 2, ...).  k_pool /
 * v_pool: caller-owned device buffers of kvc_pool_bytes each (layouts above),
 * or both NULL for a host-only handle that tracks metadata without device
 * work (appends then take NULL K/V).  The pools are not cleared.  All host
 * metadata is sized here: later calls on the handle allocate nothing except
 * the pinned staging of tables longer than 640 entries (see kvc_attend).
 * *out receives the handle.  KVC_ERR_UNSUPPORTED for device pools with
 * head_dim != 64, page_size not a multiple of 64 or units of more than 256
 * pages. */
int kvc_create(const kvc_config* cfg, void* k_pool, void* v_pool, kvc_t** out);
/* Release the handle's host metadata (the pools stay the caller's).  Waits
 * for table uploads still in flight.  NULL is accepted. */
int kvc_destroy(kvc_t* cache);

/* Append one unit ("LingBot-Map Paged KV Cache", section 2; RFC #2727,
 * section 3.3: KV append, then eviction of the oldest chunk beyond the
 * window).  k_unit / v_unit: device [patch_tokens + special_tokens][H][d],
 * patch tokens first, in the cache dtype (bf16 for FP8 caches, quantised by
 * the append); both NULL on a host-only handle.  Both 16-byte aligned
 * (KVC_ERR_INVALID_ARGUMENT otherwise).
 * Plans on the host, enqueues one scatter kernel on `stream`, and only
 * then commits the plan: KVC_ERR_OUT_OF_PAGES when the free list cannot
 * supply the unit, KVC_ERR_DEVICE when the launch fails, the cache unchanged
 * in both cases. */
int kvc_append_frame(kvc_t* cache, const void* k_unit, const void* v_unit, kvc_stream_t stream);

/* Undo the last append exactly ("LingBot-Map Paged KV Cache", section 3: a
 * non-keyframe is appended, attended, then rolled back).  Host-only: evicted
 * pages were never overwritten, so no device work is needed.  Single level;
 * KVC_ERR_NO_UNDO if there is nothing to undo. */
int kvc_rollback_last_frame(kvc_t* cache);

/* Drop every unit and restore the fresh free-list order: the once-per-window
 * reset of windowed inference ("LingBot-Map Paged KV Cache", section 4;
 * kvc_windowed_append calls it).  Host-only; device pages keep their bytes. */
int kvc_reset(kvc_t* cache);

/* Visible page table ("LingBot-Map Paged KV Cache", section 2): scale pages
 * (oldest first), window pages (oldest unit first), special pages (in the
 * order they were opened).  page_ids / page_lens: host arrays of `capacity`
 * entries; page_lens[i] is the number of valid tokens in page i (P except a
 * unit's last page, full frame-aligned special pages and the last special
 * page).  *num_pages receives the count (also on KVC_ERR_BUFFER_TOO_SMALL);
 * *last_page_len receives page_lens[num_pages - 1] (0 when empty).  Either
 * output pointer except num_pages may be NULL. */
int kvc_build_visible_table(const kvc_t* cache, int32_t* page_ids, int32_t* page_lens,
                            int32_t capacity, int32_t* num_pages, int32_t* last_page_len);

/* Copy of the metadata; see kvc_state.  It exposes what the pages' invariants
 * are stated on ("LingBot-Map Paged KV Cache", section 2: patch pages constant
 * after warm-up, out-of-window pages back on the free list, special pages
 * growing one per 42 frames; section 3: a rollback restores the state).
 * KVC_ERR_BUFFER_TOO_SMALL when out->capacity < the pool's page count and any
 * array pointer is set. */
int kvc_get_state(const kvc_t* cache, kvc_state* out);

/* ------------------------------------------------------------------------ */
/* Paged attention                                                            */
/* ------------------------------------------------------------------------ */

typedef struct paged_attn_args {
  int32_t dtype;            /* kvc_dtype of q, pools and o (FP8 pools: q and o bf16) */
  int32_t num_heads;        /* H */
  int32_t head_dim;         /* d = 64 */
  int32_t page_size;        /* P, multiple of 64 */
  float sm_scale;           /* score scale; 1/sqrt(d) is the usual value */
  int32_t num_seqs;         /* independent query sequences in this call */
  int32_t total_q;          /* rows of q and o */
  int32_t max_qo_len;       /* host-known max over sequences of query rows */
  int32_t max_kv_pages;     /* host-known max over sequences of table entries */
  int32_t num_pool_pages;   /* pool capacity; table ids outside [0, num_pool_pages) are skipped */
  int32_t num_splits;       /* key-range splits per sequence: 0 = library's choice, 1 = none */
  const int32_t* qo_indptr; /* device [num_seqs + 1]: sequence s owns q rows [qo_indptr[s], qo_indptr[s+1]) */
  const int32_t* kv_indptr; /* device [num_seqs + 1]: and table entries [kv_indptr[s], kv_indptr[s+1]) */
  const int32_t* page_ids;  /* device table: page id per entry */
  const int32_t* page_lens; /* device table: valid tokens per entry, clamped to [0, P] */
  const void* q;            /* device [total_q][H][d] */
  const void* k_pool;       /* device K pool (layout above) */
  const void* v_pool;       /* device V pool (layout above) */
  void* o;                  /* device [total_q][H][d]; rows of a sequence with no keys are 0 */
  float* lse;               /* device [total_q][H] natural-log sum of exp of scaled scores, or NULL */
  void* workspace;          /* device scratch of paged_attn_workspace_size bytes (NULL if 0) */
                            /* q, k_pool, v_pool, o and workspace must be 16-byte aligned
                               (KVC_ERR_INVALID_ARGUMENT otherwise) */
  size_t workspace_bytes;
} paged_attn_args;

/* Workspace bytes paged_attn_fwd needs for these arguments: split-key partial
 * outputs and log-sum-exps.  A sequence's key range may be cut into splits
 * that run on separate workgroups and are merged by log-sum-exp weights, the
 * same merge ring attention uses across devices (RFC #2727, section 3.4:
 * ring attention over the in-window KV); the split count is chosen by a
 * model of workgroup rounds.  Enough for every table of up to max_kv_pages
 * entries per sequence.  Reads only host fields of args. */
int paged_attn_workspace_size(const paged_attn_args* args, size_t* bytes);

/* Split count paged_attn_fwd will use for these arguments (num_splits, when
 * set, clamped to [1, max_kv_pages]; else the library's choice). */
int paged_attn_num_splits(const paged_attn_args* args, int32_t* num_splits);

/* O = softmax(sm_scale * Q K^T) V per sequence and head over the tokens of
 * the sequence's table entries, no mask ("LingBot-Map Paged KV Cache",
 * sections 1-2; RFC #2727, section 1).  bf16: matrix-core products with fp32
 * accumulation and an fp32 online softmax; fp32: fp32 throughout.  Enqueued
 * on `stream`; KVC_ERR_UNSUPPORTED for shapes the kernels do not cover. */
int paged_attn_fwd(const paged_attn_args* args, kvc_stream_t stream);

/* Merge split partials: part i of row r, head h holds a normalised output
 * O_i and its log-sum-exp lse_i; writes O = sum_i exp(lse_i - lse) O_i with
 * lse = log sum_i exp(lse_i).  partial_o: device fp32 [num_parts][rows][H][d],
 * partial_lse: device fp32 [num_parts][rows][H]; o in `dtype`, lse nullable.
 * This is the combine step of attention computed over disjoint key subsets
 * (RFC #2727, section 3.4: ring attention shards the in-window KV).  Exposed
 * for testing the merge on its own; paged_attn_fwd calls it when it splits.  partial_o and o must be 16-byte aligned (KVC_ERR_INVALID_ARGUMENT
 * otherwise). */
int paged_attn_merge(int32_t dtype, int32_t num_parts, int32_t rows, int32_t num_heads, int32_t head_dim,
                     const float* partial_o, const float* partial_lse, void* o, float* lse,
                     kvc_stream_t stream);

/* One attention step of a cache: the visible table of `cache` is built on
 * the host and handed to the kernel inside its launch arguments (no table
 * upload, nothing left to reuse), then q attends to every visible token
 * ("LingBot-Map Paged KV Cache", sections 2-3: after a frame is appended its
 * queries attend to the scale, window and special pages).  q, o: device
 * [num_q][H][d] in the cache dtype; lse: device [num_q][H] fp32 or NULL;
 * sm_scale <= 0 means 1/sqrt(d).  workspace: device scratch of
 * kvc_attend_workspace_size bytes (enough for any state of this cache).
 * Tables of up to 640 entries travel in the launch arguments.  Longer ones
 * (a LingBot stream past about 23,900 frames, whose special pages keep
 * growing, "LingBot-Map Paged KV Cache", section 2) are written to pinned
 * host memory the handle owns (a ring of 16 slots, allocated on the first
 * such call) and copied asynchronously to the start of the workspace on
 * `stream`; the host waits only when a slot's copy from 16 calls earlier has
 * not yet completed. */
int kvc_attend(const kvc_t* cache, const void* q, int32_t num_q, float sm_scale, void* o, float* lse,
               void* workspace, size_t workspace_bytes, kvc_stream_t stream);
/* Workspace bytes kvc_attend and kvc_attend_subset need for num_q queries on
 * this cache, for any table it can hold (the split partials of the largest
 * split count, plus the table region when tables can exceed 640 entries). */
int kvc_attend_workspace_size(const kvc_t* cache, int32_t num_q, size_t* bytes);

/* Page-subset table ("vLLM-Omni RFC #2727: Reconstruction Engine", section
 * 3.4, KV compression: AVGGT lets each layer attend to its own random subset
 * of the KV).  Sampling is per page of the visible table.  The first
 * keep_first and the last keep_last entries are always kept (e.g. scale
 * pages as anchors, special pages, the current unit).  Of the n entries in
 * between, ceil(keep_ratio * n) are kept: those with the smallest
 * splitmix64_i(seed), the i-th output of splitmix64 seeded with `seed`
 * (Steele, Lea, Flood 2014), where i is the entry's index in the visible
 * table; ties would go to the lower index.  Kept entries stay in table order.
 * Pass a different seed per layer for AVGGT's per-layer subsets.
 * keep_ratio in (0, 1]; 1 gives the full visible table.  Output and errors
 * as kvc_build_visible_table: *num_pages is set even when capacity is too
 * small (KVC_ERR_BUFFER_TOO_SMALL). */
int kvc_build_subset_table(const kvc_t* cache, float keep_ratio, uint64_t seed, int32_t keep_first,
                           int32_t keep_last, int32_t* page_ids, int32_t* page_lens, int32_t capacity,
                           int32_t* num_pages);
/* kvc_attend over that subset table instead of the full visible table (same
 * arguments, workspace of kvc_attend_workspace_size bytes; RFC #2727, section
 * 3.4: attention over a per-layer random KV subset). */
int kvc_attend_subset(const kvc_t* cache, float keep_ratio, uint64_t seed, int32_t keep_first, int32_t keep_last,
                      const void* q, int32_t num_q, float sm_scale, void* o, float* lse, void* workspace,
                      size_t workspace_bytes, kvc_stream_t stream);

/* One attention step of several caches in one launch: the scheduler of the
 * vLLM-Omni RFC #2727 (sections 3.2-3.3) batches the current chunks of
 * several requests; here every cache is one request or stream.  Cache i's
 * queries are rows qo_indptr[i] .. qo_indptr[i+1]-1 of q, and they attend to
 * cache i's visible table exactly as in kvc_attend.
 *
 * caches: num_caches handles (1..16) with equal num_heads, head_dim,
 * page_size and dtype.  Their pools must lie in one shared K allocation and
 * one shared V allocation: each cache's K pool starts a whole number of pages
 * after the lowest K pool pointer of the batch, and its V pool the same
 * number of pages after the lowest V pool pointer (pools handed to
 * kvc_create as page-aligned slices of two big buffers).  The combined tables
 * travel in the launch arguments: at most 640 entries in total, else
 * KVC_ERR_UNSUPPORTED (split the batch).
 * qo_indptr: host array of num_caches + 1 non-decreasing offsets, first 0.
 * q, o: device [qo_indptr[num_caches]][H][d] in the cache dtype; lse: device
 * [..][H] fp32 or NULL; sm_scale <= 0 means 1/sqrt(d).  workspace: device
 * scratch of kvc_attend_batch_workspace_size bytes for the same arguments
 * (it depends on the caches' current table lengths).
 * Errors: KVC_ERR_INVALID_ARGUMENT for mismatched configs, pools outside a
 * shared allocation, host-only caches or bad offsets; nothing is launched
 * then.  The caches are not modified. */
int kvc_attend_batch(const kvc_t* const* caches, int32_t num_caches, const void* q, const int32_t* qo_indptr,
                     float sm_scale, void* o, float* lse, void* workspace, size_t workspace_bytes,
                     kvc_stream_t stream);
/* Workspace bytes kvc_attend_batch needs for these caches in their current
 * state and these query offsets (RFC #2727, sections 3.2-3.3). */
int kvc_attend_batch_workspace_size(const kvc_t* const* caches, int32_t num_caches, const int32_t* qo_indptr,
                                    size_t* bytes);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): kvc_attend
 * without a workspace argument.  The split partials live in a device array
 * inside the library, KVC_NOALLOC_SCRATCH_BYTES (32 MiB) on each GPU it runs
 * on, held until the process ends; its address is looked up once per device
 * (on the first call made with that device current).  Nothing is allocated:
 * no device memory, no pinned staging, no host heap.
 *   - Tables must travel in the launch arguments: more than 640 visible
 *     entries gives KVC_ERR_UNSUPPORTED (use kvc_attend).
 *   - The split count is kvc_attend's whenever its partials fit the array
 *     (then results are identical to kvc_attend's); otherwise the largest
 *     split count whose partials fit is used (one split needs none), so
 *     results differ from kvc_attend's only by the rounding of the merge.
 *   - Every call on a GPU uses that GPU's one array: calls that overlap on
 *     one GPU (concurrent streams, or threads) race and give wrong results.
 *     Calls enqueued on one stream are ordered and safe.  The array needs no
 *     clearing: each call writes every partial it reads.
 *   - The current device must be the device of `stream`
 *     (KVC_ERR_INVALID_ARGUMENT otherwise).
 * Other arguments and errors as kvc_attend. */
#define KVC_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int kvc_attend_noalloc(const kvc_t* cache, const void* q, int32_t num_q, float sm_scale, void* o, float* lse,
                       kvc_stream_t stream);

/* ------------------------------------------------------------------------ */
/* Windowed inference ("LingBot-Map Paged KV Cache", section 4)              */
/* ------------------------------------------------------------------------ */

/* The page restarts the KV cache once per window of window_size KV slots
 * (stored units, not raw frames; 128 in its long run) and lets adjacent
 * windows share overlap_keyframes units.  Reading used: a slot is a kept
 * unit.  When a window holds window_slots kept units, the next append first
 * resets the cache and re-appends the last `overlap` kept units of the
 * finished window, oldest first, with the K/V they were appended with; a
 * dropped unit (keyframe skip, section 3) takes no slot.  The K/V of the last
 * `overlap` kept units wait in two caller-owned device rings of overlap + 1
 * units, so device memory stays fixed however long the stream runs: each
 * windowed append also writes its unit's K/V into the rings' free slot, in
 * the same launch as the page scatter.
 *
 * A windowed handle drives one cache; while it exists, append, roll back and
 * reset that cache only through it (attention calls on the cache are fine).
 * The cache must outlive the windowed handle. */
typedef struct kvc_windowed kvc_windowed_t;

typedef struct kvc_windowed_state {
  int32_t slots;       /* kept units in the current window */
  int32_t windows;     /* restarts so far */
  int32_t ring_units;  /* kept units waiting in the ring (at most overlap) */
  int32_t pending;     /* 1 if an appended unit waits for keep or drop */
} kvc_windowed_state;

/* Bytes of each ring (K and V) for `overlap` shared units of this cache:
 * (overlap + 1) * (patch_tokens + special_tokens) * H * d * activation
 * element size (bf16 for bf16 and FP8 caches, fp32 for fp32 caches); 0 when
 * overlap is 0 or the cache is host-only. */
int kvc_windowed_ring_bytes(const kvc_t* cache, int32_t overlap, size_t* bytes);

/* Windowed driver over `cache`.  1 <= window_slots, 0 <= overlap <
 * window_slots.  k_ring / v_ring: device buffers of kvc_windowed_ring_bytes
 * each, 16-byte aligned (NULL when overlap is 0 or the cache is host-only).
 * KVC_ERR_INVALID_ARGUMENT if the pool cannot hold window_slots + 1 units
 * (the kept units plus the one waiting for keep or drop). */
int kvc_windowed_create(kvc_t* cache, int32_t window_slots, int32_t overlap, void* k_ring, void* v_ring,
                        kvc_windowed_t** out);
int kvc_windowed_destroy(kvc_windowed_t* w);

/* Append one unit (K/V as kvc_append_frame takes them).  When the window is
 * full, first restarts it as described above; *restarted (nullable) is set to
 * 1 then, else 0.  The unit then waits for kvc_windowed_keep or
 * kvc_windowed_drop.  The append reads k_unit / v_unit in its own launch on
 * `stream` (the page scatter and the ring copy), as kvc_append_frame does.
 * Errors:
 * KVC_ERR_INVALID_ARGUMENT while a unit is waiting; if a restart fails on
 * the device, KVC_ERR_DEVICE and the windowed handle refuses every later
 * append (the cache is then part-way through a restart). */
int kvc_windowed_append(kvc_windowed_t* w, const void* k_unit, const void* v_unit, kvc_stream_t stream,
                        int32_t* restarted);
/* The waiting unit is a keyframe: it stays and takes one slot; the ring slot
 * its append wrote becomes one of the last `overlap` kept units.  Host-only
 * (no device work; `stream` is unused). */
int kvc_windowed_keep(kvc_windowed_t* w, kvc_stream_t stream);
/* The waiting unit is not kept ("LingBot-Map Paged KV Cache", section 3):
 * it is rolled back and takes no slot. */
int kvc_windowed_drop(kvc_windowed_t* w);
int kvc_windowed_get_state(const kvc_windowed_t* w, kvc_windowed_state* out);

/* ------------------------------------------------------------------------ */
/* Errors, version, measurement                                              */
/* ------------------------------------------------------------------------ */

const char* kvc_strerror(int status);
const char* kvc_last_error(void);
/* Library version as major*10000 + minor*100 + patch.  300 (0.3.0): the
 * windowed rings hold overlap + 1 units (kvc_windowed_ring_bytes), filled by
 * the windowed append itself. */
int kvc_version(void);

/* Measurement hook for timing the attention kernel apart from the host-side
 * table work and the merge of split partials: while set, every attention call
 * made on the calling thread records `start` (a hipEvent_t, or NULL) on its
 * launch stream right before the attention kernel and `done` (or NULL) right
 * after it, before the merge.  Both NULL turns it off. */
int kvc_set_kernel_events(void* start, void* done);

#ifdef __cplusplus
}
#endif

#endif /* KVC_H_ */
