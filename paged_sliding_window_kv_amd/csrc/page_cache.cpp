// Host page manager: see page_cache.hpp for the passages it follows.
#include "page_cache.hpp"

#include <algorithm>
#include <climits>

namespace kvc {

static int32_t ceil_div(int64_t a, int64_t b) { return static_cast<int32_t>((a + b - 1) / b); }

int PageCache::validate(const kvc_config& c) {
  if (c.num_heads <= 0 || c.head_dim <= 0 || c.page_size <= 0 || c.patch_tokens <= 0) return KVC_ERR_INVALID_ARGUMENT;
  if (c.special_tokens < 0 || c.special_tokens > c.page_size) return KVC_ERR_INVALID_ARGUMENT;
  if (c.num_scale_units < 0 || c.max_units <= 0 || c.num_pages < 0) return KVC_ERR_INVALID_ARGUMENT;
  if (c.dtype != KVC_DTYPE_BF16 && c.dtype != KVC_DTYPE_F32 && c.dtype != KVC_DTYPE_FP8_E4M3)
    return KVC_ERR_INVALID_ARGUMENT;
  if (c.special_packing != KVC_SPECIAL_FRAME_ALIGNED && c.special_packing != KVC_SPECIAL_CONTIGUOUS)
    return KVC_ERR_INVALID_ARGUMENT;
  return KVC_OK;
}

int32_t PageCache::required_pages(const kvc_config& c) {
  const int64_t u = ceil_div(c.patch_tokens, c.page_size);
  int64_t units = c.max_units;
  if (c.window_units > 0) units = std::min<int64_t>(units, int64_t(c.num_scale_units) + c.window_units + 1);
  int64_t special = 0;
  if (c.special_tokens > 0) {
    if (c.special_packing == KVC_SPECIAL_FRAME_ALIGNED)
      special = ceil_div(c.max_units, c.page_size / c.special_tokens);
    else
      special = ceil_div(int64_t(c.max_units) * c.special_tokens, c.page_size);
  }
  const int64_t total = units * u + special;
  return total > INT32_MAX ? -1 : static_cast<int32_t>(total);
}

PageCache::PageCache(const kvc_config& cfg) : cfg_(cfg) {
  unit_pages_ = ceil_div(cfg.patch_tokens, cfg.page_size);
  unit_tail_ = cfg.patch_tokens - cfg.page_size * (unit_pages_ - 1);
  num_pages_ = cfg.num_pages > 0 ? cfg.num_pages : required_pages(cfg);
  // Every unit holds unit_pages_ pool pages, so at most num_pages_ / unit_pages_
  // units exist at once; the window ring needs one slot more than the window
  // holds (an append pushes before it evicts, and a rollback finds the evicted
  // unit still in its slot).
  const int32_t most_units = num_pages_ / unit_pages_;
  const int32_t scale_units = std::min(cfg.num_scale_units, most_units);
  win_cap_ = most_units + 1;
  if (cfg.window_units > 0) win_cap_ = std::min(win_cap_, cfg.window_units + 1);
  free_.reserve(num_pages_);
  scale_.reserve(static_cast<size_t>(scale_units) * unit_pages_);
  win_.assign(static_cast<size_t>(win_cap_) * unit_pages_, -1);
  special_.reserve(num_pages_);
  reset();
}

void PageCache::reset() {
  free_.resize(num_pages_);
  for (int32_t i = 0; i < num_pages_; ++i) free_[i] = num_pages_ - 1 - i;  // pops give 0, 1, 2, ...
  scale_.clear();
  win_head_ = 0;
  win_count_ = 0;
  special_.clear();
  fill_ = 0;
  n_ = 0;
  has_undo_ = false;
  undo_to_scale_ = undo_evicted_ = false;
  undo_special_ = -1;
  undo_prev_fill_ = 0;
}

int32_t PageCache::frames_per_special_page() const {
  return cfg_.special_tokens > 0 ? cfg_.page_size / cfg_.special_tokens : 0;
}

int32_t PageCache::full_special_len() const {
  return cfg_.special_packing == KVC_SPECIAL_FRAME_ALIGNED ? cfg_.special_tokens * frames_per_special_page()
                                                          : cfg_.page_size;
}

// Does the next unit's special tokens need a fresh special page?  Frame
// aligned: when there is none yet or the last one holds its whole frames;
// contiguous: when the last one has less room than one unit's tokens.
bool PageCache::needs_special_page() const {
  const int32_t x = cfg_.special_tokens;
  if (x == 0) return false;
  if (special_.empty()) return true;
  if (cfg_.special_packing == KVC_SPECIAL_FRAME_ALIGNED) return fill_ == frames_per_special_page();
  return cfg_.page_size - fill_ < x;
}

int PageCache::plan(AppendPlan* plan, int32_t* unit_pages) const {
  const int32_t x = cfg_.special_tokens;
  const bool open_special = needs_special_page();
  const int32_t need = unit_pages_ + (open_special ? 1 : 0);
  if (static_cast<int32_t>(free_.size()) < need) return KVC_ERR_OUT_OF_PAGES;
  // Patch pages are popped first, then the special page.
  const size_t top = free_.size() - 1;
  if (unit_pages)
    for (int32_t i = 0; i < unit_pages_; ++i) unit_pages[i] = free_[top - i];
  const int32_t new_special = open_special ? free_[top - unit_pages_] : -1;
  if (!plan) return KVC_OK;
  *plan = AppendPlan{};
  plan->num_unit_pages = unit_pages_;
  if (x == 0) return KVC_OK;
  if (cfg_.special_packing == KVC_SPECIAL_FRAME_ALIGNED) {
    // a unit's tokens never straddle: a fresh page, or the next whole-frame slot
    plan->special_page0 = open_special ? new_special : special_.back();
    plan->special_slot0 = open_special ? 0 : x * fill_;
    plan->special_count0 = x;
  } else {
    // the room left in the last page first, the rest at the start of a fresh page
    const int32_t room = special_.empty() ? 0 : cfg_.page_size - fill_;
    const int32_t count0 = std::min(room, x);
    if (count0 > 0) {
      plan->special_page0 = special_.back();
      plan->special_slot0 = fill_;
      plan->special_count0 = count0;
      if (open_special) plan->special_page1 = new_special;
    } else {
      plan->special_page0 = new_special;
      plan->special_slot0 = 0;
      plan->special_count0 = x;
    }
  }
  return KVC_OK;
}

void PageCache::commit() {
  const int32_t x = cfg_.special_tokens;
  const bool open_special = needs_special_page();
  const int32_t room = special_.empty() ? 0 : cfg_.page_size - fill_;  // contiguous packing
  undo_prev_fill_ = fill_;
  undo_special_ = -1;
  undo_evicted_ = false;
  undo_to_scale_ = n_ < cfg_.num_scale_units;
  // Pop the unit's pages straight into their stream.
  int32_t* dst;
  if (undo_to_scale_) {
    const size_t at = scale_.size();
    scale_.resize(at + unit_pages_);  // within the reserved capacity
    dst = scale_.data() + at;
  } else {
    dst = window_slot(win_count_);
    ++win_count_;
  }
  for (int32_t i = 0; i < unit_pages_; ++i) {
    dst[i] = free_.back();
    free_.pop_back();
  }
  if (open_special) {
    undo_special_ = free_.back();
    free_.pop_back();
    special_.push_back(undo_special_);
  }
  if (x > 0) {
    if (cfg_.special_packing == KVC_SPECIAL_FRAME_ALIGNED) {
      fill_ = open_special ? 1 : fill_ + 1;
    } else {
      // contiguous: the tokens that did not fit the old page start the new one
      fill_ = open_special ? x - std::min(room, x) : fill_ + x;
    }
  }
  // After all pops: evict the oldest window unit beyond the window, pushing
  // its pages in reverse so that a later pop returns its first page first.
  if (!undo_to_scale_ && cfg_.window_units > 0 && win_count_ > cfg_.window_units) {
    const int32_t* e = window_unit(0);
    for (int32_t i = unit_pages_ - 1; i >= 0; --i) free_.push_back(e[i]);
    win_head_ = (win_head_ + 1) % win_cap_;
    --win_count_;
    undo_evicted_ = true;
  }
  has_undo_ = true;
  ++n_;
}

int PageCache::append() {
  if (int s = plan(nullptr, nullptr)) return s;
  commit();
  return KVC_OK;
}

int PageCache::rollback() {
  if (!has_undo_) return KVC_ERR_NO_UNDO;
  if (undo_evicted_) {
    // The evicted pages sit on top of the free stack in pop order, and the
    // unit is still in the ring slot before the head.
    free_.resize(free_.size() - unit_pages_);
    win_head_ = (win_head_ + win_cap_ - 1) % win_cap_;
    ++win_count_;
  }
  if (undo_special_ >= 0) {
    special_.pop_back();
    free_.push_back(undo_special_);
  }
  fill_ = undo_prev_fill_;
  --n_;
  const int32_t* u;
  if (undo_to_scale_) {
    u = scale_.data() + scale_.size() - unit_pages_;
  } else {
    u = window_unit(win_count_ - 1);
  }
  for (int32_t i = unit_pages_ - 1; i >= 0; --i) free_.push_back(u[i]);
  if (undo_to_scale_)
    scale_.resize(scale_.size() - unit_pages_);
  else
    --win_count_;
  has_undo_ = false;
  undo_to_scale_ = undo_evicted_ = false;
  undo_special_ = -1;
  return KVC_OK;
}

int32_t PageCache::visible_count() const {
  return static_cast<int32_t>(scale_.size()) + win_count_ * unit_pages_ + static_cast<int32_t>(special_.size());
}

void PageCache::visible_table(int32_t* ids, int32_t* lens) const {
  int32_t k = 0;
  auto put_unit = [&](const int32_t* u) {
    for (int32_t i = 0; i < unit_pages_; ++i) {
      if (ids) ids[k] = u[i];
      if (lens) lens[k] = (i == unit_pages_ - 1) ? unit_tail_ : cfg_.page_size;
      ++k;
    }
  };
  for (size_t i = 0; i < scale_.size(); i += unit_pages_) put_unit(scale_.data() + i);
  for (int32_t i = 0; i < win_count_; ++i) put_unit(window_unit(i));
  const int32_t full = full_special_len();
  const int32_t last = cfg_.special_packing == KVC_SPECIAL_FRAME_ALIGNED ? cfg_.special_tokens * fill_ : fill_;
  for (size_t i = 0; i < special_.size(); ++i) {
    if (ids) ids[k] = special_[i];
    if (lens) lens[k] = (i + 1 == special_.size()) ? last : full;
    ++k;
  }
}

void PageCache::state(kvc_state* st) const {
  st->num_free = static_cast<int32_t>(free_.size());
  st->num_scale_pages = static_cast<int32_t>(scale_.size());
  st->num_window_pages = win_count_ * unit_pages_;
  st->num_window_units = win_count_;
  st->num_special_pages = static_cast<int32_t>(special_.size());
  st->special_fill = fill_;
  st->num_units = n_;
  st->has_undo = has_undo_ ? 1 : 0;
  st->num_pages = num_pages_;
  if (st->free_pages) std::copy(free_.begin(), free_.end(), st->free_pages);
  if (st->scale_pages) std::copy(scale_.begin(), scale_.end(), st->scale_pages);
  if (st->window_pages) {
    int32_t k = 0;
    for (int32_t i = 0; i < win_count_; ++i) {
      const int32_t* u = window_unit(i);
      for (int32_t j = 0; j < unit_pages_; ++j) st->window_pages[k++] = u[j];
    }
  }
  if (st->special_pages) std::copy(special_.begin(), special_.end(), st->special_pages);
}

}  // namespace kvc
