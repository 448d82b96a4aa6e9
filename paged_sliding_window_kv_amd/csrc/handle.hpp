// Internal pieces shared by the C ABI sources: the cache handle, the
// thread-local error message and the exception barrier of every entry point.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <exception>
#include <new>

#include "kvc.h"
#include "page_cache.hpp"

namespace kvc {

// Pinned host staging for visible tables too long for the launch arguments:
// a ring of slots, each holding one table (ids, lens, then the two index
// pairs) that is copied asynchronously into the caller's workspace.  A slot
// is written again only after the event recorded behind its copy completed.
struct TableRing {
  static constexpr int kSlots = 16;
  int32_t* host = nullptr;      // kSlots * slot_words int32, from hipHostMalloc
  size_t slot_words = 0;
  hipEvent_t done[kSlots] = {};
  bool in_flight[kSlots] = {};
  int next = 0;
  ~TableRing();
  // Slot for the next copy, waiting for its previous copy if still in flight.
  // Allocates on first use.  Returns null on failure (message set).
  int32_t* acquire(size_t words, int* slot);
};

}  // namespace kvc

struct kvc_cache {
  kvc::PageCache pc;
  void* k_pool;
  void* v_pool;
  mutable kvc::TableRing ring;  // staging for long tables (used by const attention calls)
  explicit kvc_cache(const kvc_config& c) : pc(c), k_pool(nullptr), v_pool(nullptr) {}
};

namespace kvc {

// Sets the thread-local message kvc_last_error() returns; returns `status`.
int fail(int status, const char* fmt, ...) noexcept __attribute__((format(printf, 2, 3)));

// Runs the body of an extern "C" entry point; no exception leaves it.
template <class F>
int guarded(const char* where, F&& body) noexcept {
  try {
    return body();
  } catch (const std::bad_alloc&) {
    return fail(KVC_ERR_HOST_MEMORY, "%s: out of host memory", where);
  } catch (const std::exception& e) {
    return fail(KVC_ERR_INTERNAL, "%s: %s", where, e.what());
  } catch (...) {
    return fail(KVC_ERR_INTERNAL, "%s: unknown exception", where);
  }
}

// kvc_attend over a caller-given workspace of workspace_bytes, allocating
// nothing: only tables that travel in the launch arguments (up to 640
// entries), and the split count is lowered until the partials fit.
int attend_fixed_workspace(const kvc_t* c, const void* q, int32_t num_q, float sm_scale, void* o, float* lse,
                           void* workspace, size_t workspace_bytes, kvc_stream_t stream);

// kvc_append_frame's body; k_copy / v_copy (both or neither, device caches
// only) also receive the unit's K/V activations unchanged, in the same launch.
int append_unit(kvc_t* c, const void* k_unit, const void* v_unit, kvc_stream_t stream, void* k_copy, void* v_copy);

// Element bytes of appended K/V activations (FP8 caches take bf16).
inline size_t activation_bytes(int dtype) { return dtype == KVC_DTYPE_F32 ? 4 : 2; }

}  // namespace kvc
