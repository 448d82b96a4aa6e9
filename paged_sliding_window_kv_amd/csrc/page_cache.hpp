// Host-side page manager of one layer's paged KV cache (no device code).
//
// Implements the three page streams of "LingBot-Map Paged KV Cache",
// section 2 (scale pages kept forever, sliding-window patch pages recycled
// through a free list, append-only special pages packing many frames' special
// tokens), the scale -> window -> special visible table with per-page valid
// lengths, and the exact single-level rollback of section 3.  Units may be
// chunks of frames ("vLLM-Omni RFC #2727: Reconstruction Engine", sections 1
// and 2.3: the window keeps the most recent sliding_window_num chunks).
//
// All storage is sized at construction: plan, commit, rollback, reset and the
// table and state queries allocate nothing and cannot throw.
#pragma once

#include <cstdint>
#include <vector>

#include "kvc.h"

namespace kvc {

// Where one append puts its tokens; consumed by the scatter kernel.
struct AppendPlan {
  int32_t num_unit_pages = 0;       // patch token i -> (unit page i / P, slot i % P)
  int32_t special_page0 = -1;       // special token j < special_count0 -> (special_page0, special_slot0 + j)
  int32_t special_slot0 = 0;
  int32_t special_count0 = 0;
  int32_t special_page1 = -1;       // special token j >= special_count0 -> (special_page1, j - special_count0)
};

class PageCache {
 public:
  explicit PageCache(const kvc_config& cfg);

  const kvc_config& config() const { return cfg_; }
  int32_t num_pages() const { return num_pages_; }
  int32_t unit_pages() const { return unit_pages_; }

  // Plans the next append without changing any state: fills *plan and, when
  // unit_pages is not null, the unit's num_unit_pages page ids.  Returns
  // KVC_OK or KVC_ERR_OUT_OF_PAGES.
  int plan(AppendPlan* plan, int32_t* unit_pages) const;
  // Applies exactly the append plan() describes (call only after plan()
  // returned KVC_OK on the unchanged cache).
  void commit();
  // plan() then commit().
  int append();
  // Undoes the last append.  KVC_ERR_NO_UNDO when there is none.
  int rollback();
  void reset();

  int32_t num_units() const { return n_; }
  int32_t visible_count() const;
  // Writes visible_count() entries.
  void visible_table(int32_t* ids, int32_t* lens) const;
  void state(kvc_state* st) const;

  static int32_t required_pages(const kvc_config& cfg);
  static int validate(const kvc_config& cfg);

 private:
  int32_t frames_per_special_page() const;
  int32_t full_special_len() const;
  bool needs_special_page() const;
  // Page list of window unit i (0 = oldest) inside the ring.
  const int32_t* window_unit(int32_t i) const {
    return win_.data() + static_cast<size_t>((win_head_ + i) % win_cap_) * unit_pages_;
  }
  int32_t* window_slot(int32_t i) {
    return win_.data() + static_cast<size_t>((win_head_ + i) % win_cap_) * unit_pages_;
  }

  kvc_config cfg_;
  int32_t num_pages_ = 0;
  int32_t unit_pages_ = 0;
  int32_t unit_tail_ = 0;
  std::vector<int32_t> free_;     // stack; back() is the next page popped (capacity num_pages_)
  std::vector<int32_t> scale_;    // scale units' pages in order, unit_pages_ per unit
  std::vector<int32_t> win_;      // ring of win_cap_ window units, unit_pages_ pages each
  int32_t win_cap_ = 0;
  int32_t win_head_ = 0;          // ring slot of the oldest window unit
  int32_t win_count_ = 0;
  std::vector<int32_t> special_;  // special pages in the order they were opened
  int32_t fill_ = 0;
  int32_t n_ = 0;
  // Undo record of the last append (single level).
  bool has_undo_ = false;
  bool undo_to_scale_ = false;
  bool undo_evicted_ = false;
  int32_t undo_special_ = -1;     // special page the append opened, or -1
  int32_t undo_prev_fill_ = 0;
};

}  // namespace kvc
