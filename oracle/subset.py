"""Page-subset visible tables (test infrastructure: the oracle of the subset tables).

"vLLM-Omni RFC #2727: Reconstruction Engine", section 3.4, item 3 (KV
compression), lists AVGGT: every layer attends to a random subset of the KV,
different layers drawing different subsets, with a keep ratio of 0.25 in the
medium-scale configuration of the same section.  Reading used here (the pages
fix neither the granularity nor the generator): sampling is per page of the
visible table.  An optional leading run (keep_first entries, e.g. the scale
pages) and trailing run (keep_last entries, e.g. the special pages or the
current unit) are always kept.  From the n remaining candidate entries,
m = ceil(keep_ratio * n) are kept: those whose keys are smallest.  Entry i of
the table gets the key splitmix64_i(seed), the i-th output (counting from 0)
of the splitmix64 generator seeded with `seed`.  Ties would break on the
index.  Kept entries stay in table order.

splitmix64 is Steele, Lea and Flood's generator (OOPSLA 2014, "Fast
splittable pseudorandom number generators"), in the public reference form:
the state advances by the golden-ratio constant 0x9E3779B97F4A7C15, and the
output is the state after three xor-shift / multiply rounds.
"""
from __future__ import annotations

import math
from typing import List, Sequence, Tuple

_M64 = (1 << 64) - 1
_GOLDEN = 0x9E3779B97F4A7C15


def splitmix64(seed: int, i: int) -> int:
    """The i-th output (0-based) of splitmix64 seeded with `seed`."""
    z = (seed + (i + 1) * _GOLDEN) & _M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _M64
    return z ^ (z >> 31)


def subset_keep_count(n: int, keep_ratio: float) -> int:
    """Candidates kept out of n: ceil(keep_ratio * n), evaluated in float32 as the library's argument is."""
    import numpy as np
    if n <= 0:
        return 0
    return min(n, int(math.ceil(float(np.float32(keep_ratio)) * n)))


def subset_table(ids: Sequence[int], lens: Sequence[int], keep_ratio: float, seed: int, keep_first: int = 0,
                 keep_last: int = 0) -> Tuple[List[int], List[int]]:
    """The page subset of a visible table (ids, lens) under the reading above."""
    if not (0.0 < keep_ratio <= 1.0):
        raise ValueError("keep_ratio must be in (0, 1]")
    n = len(ids)
    kf = max(0, min(keep_first, n))
    kl = max(0, min(keep_last, n - kf))
    cand = list(range(kf, n - kl))
    m = subset_keep_count(len(cand), keep_ratio)
    ranked = sorted(cand, key=lambda i: (splitmix64(seed & _M64, i), i))
    kept = set(range(kf)) | set(range(n - kl, n)) | set(ranked[:m])
    order = [i for i in range(n) if i in kept]
    return [ids[i] for i in order], [lens[i] for i in order]
