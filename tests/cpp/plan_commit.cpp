// Host check of the page manager's plan/commit split: plan() changes nothing
// (so an append whose scatter fails to launch leaves the cache, and the undo
// record of the previous append, exactly as they were), and commit() applies
// exactly the planned pages.  Built and run by tests/test_plan_commit.py.
#include <cstdio>
#include <cstring>
#include <vector>

#include "page_cache.hpp"

namespace {

// Visible table, page lists (free stack, scale, window, special) and counts.
struct Snapshot {
  std::vector<int32_t> ids, lens, lists, counts;
};

Snapshot snap(const kvc::PageCache& pc) {
  Snapshot s;
  const int32_t n = pc.visible_count();
  s.ids.resize(n);
  s.lens.resize(n);
  pc.visible_table(s.ids.data(), s.lens.data());
  const int32_t cap = pc.num_pages();
  std::vector<int32_t> fr(cap), sc(cap), wi(cap), sp(cap);
  kvc_state st;
  std::memset(&st, 0, sizeof st);
  st.capacity = cap;
  st.free_pages = fr.data();
  st.scale_pages = sc.data();
  st.window_pages = wi.data();
  st.special_pages = sp.data();
  pc.state(&st);
  s.counts = {st.num_free, st.num_scale_pages, st.num_window_pages, st.num_window_units, st.num_special_pages,
              st.special_fill, st.num_units, st.has_undo, st.num_pages};
  s.lists.insert(s.lists.end(), fr.begin(), fr.begin() + st.num_free);
  s.lists.push_back(-1);
  s.lists.insert(s.lists.end(), sc.begin(), sc.begin() + st.num_scale_pages);
  s.lists.push_back(-1);
  s.lists.insert(s.lists.end(), wi.begin(), wi.begin() + st.num_window_pages);
  s.lists.push_back(-1);
  s.lists.insert(s.lists.end(), sp.begin(), sp.begin() + st.num_special_pages);
  return s;
}

bool same(const Snapshot& a, const Snapshot& b) {
  return a.ids == b.ids && a.lens == b.lens && a.lists == b.lists && a.counts == b.counts;
}

int fails = 0;
void check(bool ok, const char* what, int t) {
  if (!ok) {
    std::printf("FAIL %s at frame %d\n", what, t);
    ++fails;
  }
}

}  // namespace

int main() {
  // A small LingBot-shaped layer: 4-token pages, 4 patch + 2 special tokens
  // per frame, 1 scale frame, a 2-frame window, frame-aligned special pages.
  kvc_config cfg;
  std::memset(&cfg, 0, sizeof cfg);
  cfg.num_heads = 1;
  cfg.head_dim = 64;
  cfg.page_size = 4;
  cfg.dtype = KVC_DTYPE_BF16;
  cfg.patch_tokens = 4;
  cfg.special_tokens = 2;
  cfg.num_scale_units = 1;
  cfg.window_units = 2;
  cfg.special_packing = 0;
  cfg.max_units = 40;
  cfg.num_pages = 0;
  if (kvc::PageCache::validate(cfg) != KVC_OK) {
    std::printf("FAIL config\n");
    return 1;
  }
  kvc::PageCache pc(cfg), ref(cfg);
  std::vector<int32_t> unit(pc.unit_pages());
  for (int t = 0; t < 30; ++t) {
    const Snapshot before = snap(pc);
    // A planned append that is never committed (its launch failed).
    kvc::AppendPlan plan;
    check(pc.plan(&plan, unit.data()) == KVC_OK, "plan", t);
    check(same(before, snap(pc)), "plan changed the cache", t);
    if (t > 0) {
      // The previous append's undo record survives the abandoned plan: undo
      // it on a copy and compare with the reference before that append.
      kvc::PageCache probe = pc;
      check(probe.rollback() == KVC_OK, "undo after an abandoned plan", t);
      kvc::PageCache r0 = ref;
      check(r0.rollback() == KVC_OK, "reference undo", t);
      check(same(snap(probe), snap(r0)), "undo after an abandoned plan differs", t);
    }
    // Plan again and commit: the same pages as plan() reported, and the same
    // cache as a plain append.
    kvc::AppendPlan plan2;
    std::vector<int32_t> unit2(pc.unit_pages());
    check(pc.plan(&plan2, unit2.data()) == KVC_OK, "replan", t);
    check(unit == unit2 && plan.special_page0 == plan2.special_page0 && plan.special_slot0 == plan2.special_slot0 &&
              plan.special_count0 == plan2.special_count0 && plan.special_page1 == plan2.special_page1,
          "plan not deterministic", t);
    pc.commit();
    check(ref.append() == KVC_OK, "reference append", t);
    check(same(snap(pc), snap(ref)), "commit differs from append", t);
    // The committed unit's pages are the planned ones: they are the newest
    // window (or scale) entries of the visible table.
    const Snapshot after = snap(pc);
    bool found = true;
    for (int32_t id : unit) {
      bool in = false;
      for (int32_t v : after.ids) in = in || v == id;
      found = found && in;
    }
    check(found, "planned pages not visible", t);
  }
  if (fails == 0) std::printf("OK plan/commit 30 frames\n");
  return fails == 0 ? 0 : 1;
}
