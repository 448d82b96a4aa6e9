// Page-subset visible tables: per-layer random page sampling of the visible
// table ("vLLM-Omni RFC #2727: Reconstruction Engine", section 3.4, KV
// compression: AVGGT samples a random KV subset per layer).
#pragma once

#include <cstdint>

namespace kvc {

// The i-th output (0-based) of the splitmix64 generator seeded with `seed`
// (Steele, Lea, Flood, OOPSLA 2014; public reference form).
uint64_t splitmix64(uint64_t seed, uint64_t i);

// Candidates kept out of n: ceil(keep_ratio * n), at most n.
int32_t subset_keep_count(int32_t n, float keep_ratio);

// Writes the subset of the table (ids, lens; n entries) to out_ids/out_lens
// (room for n entries) and returns its length.  The first keep_first and last
// keep_last entries are always kept; of the others, the subset_keep_count
// ones with the smallest splitmix64_i(seed) (ties on i) are kept.  Kept
// entries stay in table order.  keep_ratio must be in (0, 1].
int32_t subset_select(const int32_t* ids, const int32_t* lens, int32_t n, float keep_ratio, uint64_t seed,
                      int32_t keep_first, int32_t keep_last, int32_t* out_ids, int32_t* out_lens);

}  // namespace kvc
