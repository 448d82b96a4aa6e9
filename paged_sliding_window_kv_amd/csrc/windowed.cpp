// Windowed inference over one cache ("LingBot-Map Paged KV Cache", section 4;
// declared in include/kvc.h).
//
// The page restarts the KV cache once per window of window_size KV slots
// (stored units, not raw frames) and lets adjacent windows share
// overlap_keyframes units.  Reading used (the page fixes neither the order nor
// where the shared units' K/V come from): a slot is a kept unit; when a window
// holds window_slots kept units, the next append first resets the cache and
// re-appends the last `overlap` kept units of the finished window, oldest
// first, with the K/V they were appended with.  Units that are dropped (a
// keyframe skip rolls them back) take no slot.  The K/V of the last `overlap`
// kept units wait in a caller-owned device ring, so device memory stays fixed
// however long the stream runs.  The ring has one slot more than `overlap`:
// every windowed append writes its unit's K/V into the free slot in the same
// launch that scatters them into pages, and keeping the unit only advances
// the ring (no copy of its own), while a dropped unit's slot is simply written
// again by the next append.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "handle.hpp"
#include "kvc.h"
#include "page_cache.hpp"

using kvc::fail;
using kvc::guarded;

struct kvc_windowed {
  kvc_t* cache = nullptr;
  int32_t window_slots = 0;
  int32_t overlap = 0;
  char* k_ring = nullptr;  // device [overlap + 1][unit tokens][H][d] activations, or null (host-only cache)
  char* v_ring = nullptr;
  size_t unit_bytes = 0;
  int32_t slots = 0;       // kept units in the current window
  int32_t windows = 0;     // restarts so far
  int32_t ring_len = 0;    // kept units in the ring (at most overlap)
  int32_t ring_head = 0;   // the free slot: the next append's K/V go here
  bool pending = false;    // an appended unit waits for keep or drop
  bool broken = false;     // a restart failed part-way on the device
};

namespace {

size_t unit_activation_bytes(const kvc_config& c) {
  return static_cast<size_t>(c.patch_tokens + c.special_tokens) * c.num_heads * c.head_dim *
         kvc::activation_bytes(c.dtype);
}

int32_t ring_slots(const kvc_windowed* w) { return w->overlap > 0 ? w->overlap + 1 : 0; }

// Restart: reset the cache and re-append the ring's units, oldest first.
int restart(kvc_windowed* w, kvc_stream_t stream) {
  if (int s = kvc_reset(w->cache)) return s;
  const int32_t r = ring_slots(w);
  for (int32_t j = 0; j < w->ring_len; ++j) {
    const int32_t slot = ((w->ring_head - w->ring_len + j) % r + r) % r;
    const void* k = w->k_ring ? w->k_ring + slot * w->unit_bytes : nullptr;
    const void* v = w->v_ring ? w->v_ring + slot * w->unit_bytes : nullptr;
    if (int s = kvc_append_frame(w->cache, k, v, stream)) {
      w->broken = true;
      return s;
    }
  }
  w->slots = w->ring_len;
  ++w->windows;
  return KVC_OK;
}

}  // namespace

extern "C" {

int kvc_windowed_ring_bytes(const kvc_t* cache, int32_t overlap, size_t* bytes) {
  return guarded("kvc_windowed_ring_bytes", [&] {
    if (!cache || !bytes || overlap < 0) return fail(KVC_ERR_INVALID_ARGUMENT, "bad argument");
    const size_t slots = overlap > 0 ? static_cast<size_t>(overlap) + 1 : 0;
    *bytes = cache->k_pool ? slots * unit_activation_bytes(cache->pc.config()) : 0;
    return static_cast<int>(KVC_OK);
  });
}

int kvc_windowed_create(kvc_t* cache, int32_t window_slots, int32_t overlap, void* k_ring, void* v_ring,
                        kvc_windowed_t** out) {
  return guarded("kvc_windowed_create", [&] {
    if (!cache || !out) return fail(KVC_ERR_INVALID_ARGUMENT, "NULL argument");
    if (window_slots < 1 || overlap < 0 || overlap >= window_slots)
      return fail(KVC_ERR_INVALID_ARGUMENT, "need window_slots >= 1 and 0 <= overlap < window_slots");
    const bool device = cache->k_pool != nullptr;
    if (device && overlap > 0 && (!k_ring || !v_ring))
      return fail(KVC_ERR_INVALID_ARGUMENT, "a device cache with overlap > 0 needs K and V rings");
    if (!device && (k_ring || v_ring)) return fail(KVC_ERR_INVALID_ARGUMENT, "a host-only cache takes no rings");
    if ((reinterpret_cast<uintptr_t>(k_ring) | reinterpret_cast<uintptr_t>(v_ring)) & 15)
      return fail(KVC_ERR_INVALID_ARGUMENT, "rings must be 16-byte aligned");
    // A window holds window_slots kept units plus the unit waiting for keep or
    // drop: the pool must fit that many units at any point of the stream.
    kvc_config need = cache->pc.config();
    need.max_units = window_slots + 1;
    need.num_pages = 0;
    const int32_t pages = kvc::PageCache::required_pages(need);
    if (pages < 0 || pages > cache->pc.num_pages())
      return fail(KVC_ERR_INVALID_ARGUMENT, "the pool holds %d pages; a window of %d slots needs %d",
                  cache->pc.num_pages(), window_slots, pages);
    kvc_windowed* w = new kvc_windowed;
    w->cache = cache;
    w->window_slots = window_slots;
    w->overlap = overlap;
    w->k_ring = static_cast<char*>(k_ring);
    w->v_ring = static_cast<char*>(v_ring);
    w->unit_bytes = unit_activation_bytes(cache->pc.config());
    *out = w;
    return static_cast<int>(KVC_OK);
  });
}

int kvc_windowed_destroy(kvc_windowed_t* w) {
  return guarded("kvc_windowed_destroy", [&] {
    delete w;
    return static_cast<int>(KVC_OK);
  });
}

int kvc_windowed_append(kvc_windowed_t* w, const void* k_unit, const void* v_unit, kvc_stream_t stream,
                        int32_t* restarted) {
  return guarded("kvc_windowed_append", [&] {
    if (!w) return fail(KVC_ERR_INVALID_ARGUMENT, "NULL handle");
    if (restarted) *restarted = 0;
    if (w->broken) return fail(KVC_ERR_DEVICE, "a restart of this windowed stream failed on the device");
    if (w->pending) return fail(KVC_ERR_INVALID_ARGUMENT, "keep or drop the previous unit first");
    const bool device = w->cache->k_pool != nullptr;
    if (device != (k_unit != nullptr) || device != (v_unit != nullptr))
      return fail(KVC_ERR_INVALID_ARGUMENT, device ? "device cache needs K and V" : "host-only cache takes NULL K/V");
    if ((reinterpret_cast<uintptr_t>(k_unit) | reinterpret_cast<uintptr_t>(v_unit)) & 15)
      return fail(KVC_ERR_INVALID_ARGUMENT, "K and V must be 16-byte aligned");
    if (w->slots >= w->window_slots) {
      if (int s = restart(w, stream)) return s;
      if (restarted) *restarted = 1;
    }
    // the unit's K/V also go to the ring's free slot, in the append's own launch
    char* kc = nullptr;
    char* vc = nullptr;
    if (w->overlap > 0 && w->k_ring) {
      const size_t off = static_cast<size_t>(w->ring_head) * w->unit_bytes;
      kc = w->k_ring + off;
      vc = w->v_ring + off;
    }
    if (int s = kvc::append_unit(w->cache, k_unit, v_unit, stream, kc, vc)) return s;
    w->pending = true;
    return static_cast<int>(KVC_OK);
  });
}

int kvc_windowed_keep(kvc_windowed_t* w, kvc_stream_t stream) {
  (void)stream;  // the append already placed the unit's K/V in the ring's free slot
  return guarded("kvc_windowed_keep", [&] {
    if (!w) return fail(KVC_ERR_INVALID_ARGUMENT, "NULL handle");
    if (!w->pending) return fail(KVC_ERR_INVALID_ARGUMENT, "nothing appended");
    if (w->overlap > 0) {
      // the slot written by the append now holds the newest kept unit; the
      // next free slot held the unit kept overlap + 1 keeps ago
      w->ring_head = (w->ring_head + 1) % ring_slots(w);
      w->ring_len = std::min(w->ring_len + 1, w->overlap);
    }
    ++w->slots;
    w->pending = false;
    return static_cast<int>(KVC_OK);
  });
}

int kvc_windowed_drop(kvc_windowed_t* w) {
  return guarded("kvc_windowed_drop", [&] {
    if (!w) return fail(KVC_ERR_INVALID_ARGUMENT, "NULL handle");
    if (!w->pending) return fail(KVC_ERR_INVALID_ARGUMENT, "nothing appended");
    if (int s = kvc_rollback_last_frame(w->cache)) return s;
    w->pending = false;
    return static_cast<int>(KVC_OK);
  });
}

int kvc_windowed_get_state(const kvc_windowed_t* w, kvc_windowed_state* st) {
  return guarded("kvc_windowed_get_state", [&] {
    if (!w || !st) return fail(KVC_ERR_INVALID_ARGUMENT, "NULL argument");
    st->slots = w->slots;
    st->windows = w->windows;
    st->ring_units = w->ring_len;
    st->pending = w->pending ? 1 : 0;
    return static_cast<int>(KVC_OK);
  });
}

}  // extern "C"
