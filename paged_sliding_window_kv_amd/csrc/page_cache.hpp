// Host-side page manager of one layer's paged KV cache (no device code).
//
// Implements the three page streams of "LingBot-Map Paged KV Cache",
// section 2 (scale pages kept forever, sliding-window patch pages recycled
// through a free list, append-only special pages packing many frames' special
// tokens), the scale -> window -> special visible table with per-page valid
// lengths, and the exact single-level rollback of section 3.  Units may be
// chunks of frames ("vLLM-Omni RFC #2727: Reconstruction Engine", sections 1
// and 2.3: the window keeps the most recent sliding_window_num chunks).
#pragma once

#include <cstdint>
#include <deque>
#include <vector>

#include "kvc.h"

namespace kvc {

// Where one append puts its tokens; consumed by the scatter kernel.
struct AppendPlan {
  std::vector<int32_t> unit_pages;  // patch token i -> (unit_pages[i / P], i % P)
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

  // Plans and commits one append.  Returns KVC_OK or KVC_ERR_OUT_OF_PAGES
  // (state unchanged).
  int append(AppendPlan* plan);
  // Undoes the last append.  KVC_ERR_NO_UNDO when there is none.
  int rollback();
  void reset();

  int32_t visible_count() const;
  // Writes visible_count() entries.
  void visible_table(int32_t* ids, int32_t* lens) const;
  void state(kvc_state* st) const;

  static int32_t required_pages(const kvc_config& cfg);
  static int validate(const kvc_config& cfg);

 private:
  struct Undo {
    std::vector<int32_t> unit;
    std::vector<int32_t> evicted;
    bool has_evicted = false;
    int32_t new_special = -1;
    int32_t prev_fill = 0;
    bool to_scale = false;
  };

  int32_t frames_per_special_page() const;
  int32_t full_special_len() const;

  kvc_config cfg_;
  int32_t num_pages_ = 0;
  int32_t unit_pages_ = 0;
  int32_t unit_tail_ = 0;
  std::vector<int32_t> free_;  // stack; back() is the next page popped
  std::vector<std::vector<int32_t>> scale_;
  std::deque<std::vector<int32_t>> window_;
  std::vector<int32_t> special_;
  int32_t fill_ = 0;
  int32_t n_ = 0;
  bool has_undo_ = false;
  Undo undo_;
};

}  // namespace kvc
