// Host page manager: see page_cache.hpp for the passages it follows.
#include "page_cache.hpp"

#include <algorithm>

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
  reset();
}

void PageCache::reset() {
  free_.resize(num_pages_);
  for (int32_t i = 0; i < num_pages_; ++i) free_[i] = num_pages_ - 1 - i;  // pops give 0, 1, 2, ...
  scale_.clear();
  window_.clear();
  special_.clear();
  fill_ = 0;
  n_ = 0;
  has_undo_ = false;
  undo_ = Undo{};
}

int32_t PageCache::frames_per_special_page() const {
  return cfg_.special_tokens > 0 ? cfg_.page_size / cfg_.special_tokens : 0;
}

int32_t PageCache::full_special_len() const {
  return cfg_.special_packing == KVC_SPECIAL_FRAME_ALIGNED ? cfg_.special_tokens * frames_per_special_page()
                                                          : cfg_.page_size;
}

int PageCache::append(AppendPlan* plan) {
  const int32_t x = cfg_.special_tokens;
  const int32_t page = cfg_.page_size;
  // Where do this unit's special tokens go, and is a new special page needed?
  bool open_special = false;
  int32_t slot0 = 0, count0 = 0;
  if (x > 0) {
    if (cfg_.special_packing == KVC_SPECIAL_FRAME_ALIGNED) {
      open_special = special_.empty() || fill_ == frames_per_special_page();
      slot0 = open_special ? 0 : x * fill_;
      count0 = x;
    } else {
      const int32_t room = special_.empty() ? 0 : page - fill_;
      open_special = room < x;
      count0 = std::min(room, x);
      slot0 = special_.empty() ? 0 : fill_;
    }
  }
  const int32_t need = unit_pages_ + (open_special ? 1 : 0);
  if (static_cast<int32_t>(free_.size()) < need) return KVC_ERR_OUT_OF_PAGES;

  // Patch pages first, then the special page.
  std::vector<int32_t> unit(unit_pages_);
  for (int32_t i = 0; i < unit_pages_; ++i) {
    unit[i] = free_.back();
    free_.pop_back();
  }
  Undo ud;
  ud.prev_fill = fill_;
  if (open_special) {
    ud.new_special = free_.back();
    free_.pop_back();
    special_.push_back(ud.new_special);
  }
  if (plan) {
    plan->unit_pages = unit;
    plan->special_page0 = plan->special_page1 = -1;
    plan->special_slot0 = plan->special_count0 = 0;
    if (x > 0) {
      if (cfg_.special_packing == KVC_SPECIAL_FRAME_ALIGNED) {
        plan->special_page0 = special_.back();
        plan->special_slot0 = slot0;
        plan->special_count0 = x;
      } else if (count0 > 0) {
        const size_t cur = special_.size() - (open_special ? 2 : 1);
        plan->special_page0 = special_[cur];
        plan->special_slot0 = slot0;
        plan->special_count0 = count0;
        if (open_special) plan->special_page1 = special_.back();
      } else {
        plan->special_page0 = special_.back();
        plan->special_slot0 = 0;
        plan->special_count0 = x;
      }
    }
  }
  if (x > 0) {
    if (cfg_.special_packing == KVC_SPECIAL_FRAME_ALIGNED)
      fill_ = open_special ? 1 : fill_ + 1;
    else
      fill_ = open_special ? x - count0 : fill_ + x;
  }
  ud.to_scale = n_ < cfg_.num_scale_units;
  if (ud.to_scale) {
    scale_.push_back(unit);
  } else {
    window_.push_back(unit);
    if (cfg_.window_units > 0 && static_cast<int32_t>(window_.size()) > cfg_.window_units) {
      ud.evicted = std::move(window_.front());
      ud.has_evicted = true;
      window_.pop_front();
      for (auto it = ud.evicted.rbegin(); it != ud.evicted.rend(); ++it) free_.push_back(*it);
    }
  }
  ud.unit = std::move(unit);
  undo_ = std::move(ud);
  has_undo_ = true;
  ++n_;
  return KVC_OK;
}

int PageCache::rollback() {
  if (!has_undo_) return KVC_ERR_NO_UNDO;
  Undo& ud = undo_;
  if (ud.has_evicted) {
    // The evicted pages sit on top of the free stack in pop order.
    free_.resize(free_.size() - ud.evicted.size());
    window_.push_front(std::move(ud.evicted));
  }
  if (ud.new_special >= 0) {
    special_.pop_back();
    free_.push_back(ud.new_special);
  }
  fill_ = ud.prev_fill;
  --n_;
  if (ud.to_scale)
    scale_.pop_back();
  else
    window_.pop_back();
  for (auto it = ud.unit.rbegin(); it != ud.unit.rend(); ++it) free_.push_back(*it);
  has_undo_ = false;
  undo_ = Undo{};
  return KVC_OK;
}

int32_t PageCache::visible_count() const {
  return static_cast<int32_t>((scale_.size() + window_.size()) * unit_pages_ + special_.size());
}

void PageCache::visible_table(int32_t* ids, int32_t* lens) const {
  int32_t k = 0;
  auto put_unit = [&](const std::vector<int32_t>& u) {
    for (int32_t i = 0; i < unit_pages_; ++i) {
      if (ids) ids[k] = u[i];
      if (lens) lens[k] = (i == unit_pages_ - 1) ? unit_tail_ : cfg_.page_size;
      ++k;
    }
  };
  for (const auto& u : scale_) put_unit(u);
  for (const auto& u : window_) put_unit(u);
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
  st->num_scale_pages = static_cast<int32_t>(scale_.size()) * unit_pages_;
  st->num_window_pages = static_cast<int32_t>(window_.size()) * unit_pages_;
  st->num_window_units = static_cast<int32_t>(window_.size());
  st->num_special_pages = static_cast<int32_t>(special_.size());
  st->special_fill = fill_;
  st->num_units = n_;
  st->has_undo = has_undo_ ? 1 : 0;
  st->num_pages = num_pages_;
  if (st->free_pages) std::copy(free_.begin(), free_.end(), st->free_pages);
  if (st->scale_pages) {
    int32_t k = 0;
    for (const auto& u : scale_)
      for (int32_t p : u) st->scale_pages[k++] = p;
  }
  if (st->window_pages) {
    int32_t k = 0;
    for (const auto& u : window_)
      for (int32_t p : u) st->window_pages[k++] = p;
  }
  if (st->special_pages) std::copy(special_.begin(), special_.end(), st->special_pages);
}

}  // namespace kvc
