// Page-subset visible tables (declared in subset.hpp).
#include "subset.hpp"

#include <algorithm>
#include <cmath>
#include <utility>
#include <vector>

namespace kvc {

uint64_t splitmix64(uint64_t seed, uint64_t i) {
  uint64_t z = seed + (i + 1) * 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

int32_t subset_keep_count(int32_t n, float keep_ratio) {
  if (n <= 0) return 0;
  const double m = std::ceil(static_cast<double>(keep_ratio) * n);
  return static_cast<int32_t>(std::min<double>(m, n));
}

int32_t subset_select(const int32_t* ids, const int32_t* lens, int32_t n, float keep_ratio, uint64_t seed,
                      int32_t keep_first, int32_t keep_last, int32_t* out_ids, int32_t* out_lens) {
  const int32_t kf = std::max(0, std::min(keep_first, n));
  const int32_t kl = std::max(0, std::min(keep_last, n - kf));
  std::vector<std::pair<uint64_t, int32_t>> cand;
  cand.reserve(static_cast<size_t>(n - kf - kl));
  for (int32_t i = kf; i < n - kl; ++i) cand.emplace_back(splitmix64(seed, static_cast<uint64_t>(i)), i);
  const int32_t m = subset_keep_count(static_cast<int32_t>(cand.size()), keep_ratio);
  std::vector<char> keep(static_cast<size_t>(n), 0);
  for (int32_t i = 0; i < kf; ++i) keep[i] = 1;
  for (int32_t i = n - kl; i < n; ++i) keep[i] = 1;
  if (m > 0) {
    std::nth_element(cand.begin(), cand.begin() + (m - 1), cand.end());
    for (int32_t j = 0; j < m; ++j) keep[cand[j].second] = 1;
  }
  int32_t k = 0;
  for (int32_t i = 0; i < n; ++i)
    if (keep[i]) {
      out_ids[k] = ids[i];
      out_lens[k] = lens[i];
      ++k;
    }
  return k;
}

}  // namespace kvc
