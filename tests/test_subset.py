"""Page-subset tables: the oracle's sampler pinned, and the library's tables bit-exact against it."""
import math

import numpy as np
import pytest

from oracle import OracleCache, OracleConfig, is_keyframe, splitmix64, subset_keep_count, subset_table
from paged_sliding_window_kv_amd import KvCache


def test_splitmix64_published_outputs():
    # First three outputs of splitmix64 seeded with 0, as published with the
    # reference implementation (Steele, Lea, Flood 2014; Vigna's C version).
    assert splitmix64(0, 0) == 0xE220A8397B1DCDAF
    assert splitmix64(0, 1) == 0x6E789E6AA1B965F4
    assert splitmix64(0, 2) == 0x06C45D188009454F


def test_subset_properties():
    ids = list(range(100, 172))
    lens = [256] * 71 + [144]
    # keep_ratio 1 is the identity
    assert subset_table(ids, lens, 1.0, 5) == (ids, lens)
    for r in (0.01, 0.25, 0.5, 0.99):
        for kf, kl in ((0, 0), (8, 3), (70, 5)):
            si, sl = subset_table(ids, lens, r, 11, kf, kl)
            n_c = max(0, len(ids) - min(kf, len(ids)) - min(kl, len(ids) - min(kf, len(ids))))
            assert len(si) == min(kf, 72) + min(kl, 72 - min(kf, 72)) + math.ceil(np.float32(r) * n_c)
            assert si == sorted(si)                       # table order kept
            assert set(ids[:kf]) <= set(si)               # leading run kept
            if kl:
                assert set(ids[len(ids) - kl:]) <= set(si)
            assert all(lens[ids.index(p)] == q for p, q in zip(si, sl))
    # deterministic per seed, different across seeds
    assert subset_table(ids, lens, 0.25, 3) == subset_table(ids, lens, 0.25, 3)
    assert subset_table(ids, lens, 0.25, 3) != subset_table(ids, lens, 0.25, 4)


def test_subset_is_uniform_over_seeds():
    """Each candidate is kept with probability m/n: frequency over 2000 seeds within 5 sigma."""
    ids = list(range(40))
    lens = [256] * 40
    trials, r = 2000, 0.25
    m = subset_keep_count(40, r)
    p = m / 40
    counts = np.zeros(40)
    for s in range(trials):
        si, _ = subset_table(ids, lens, r, 1000 + s)
        counts[si] += 1
    sigma = math.sqrt(trials * p * (1 - p))
    assert np.abs(counts - trials * p).max() < 5 * sigma


@pytest.mark.parametrize("seed", [0, 1, 2**63 + 17, 2**64 - 1])
def test_library_subset_matches_oracle(seed):
    H, P, X, S, W = 2, 256, 6, 2, 6
    oc = OracleCache(OracleConfig(num_heads=H, head_dim=64, patch_tokens=P, special_tokens=X, num_scale_units=S,
                                  window_units=W, max_units=400), with_pool=False)
    hc = KvCache(num_heads=H, patch_tokens=P, special_tokens=X, num_scale_units=S, window_units=W, max_units=400)
    rng = np.random.default_rng(seed % 1000)
    for t in range(300):
        oc.append()
        hc.append()
        if not is_keyframe(t, S, 2):
            oc.rollback()
            hc.rollback()
        if t % 37 == 0:
            ids, lens = oc.visible_table()
            for r in (1.0, 0.75, 0.25, 0.1):
                kf, kl = int(rng.integers(0, 4)), int(rng.integers(0, 4))
                want = subset_table(ids, lens, r, seed, kf, kl)
                got = hc.subset_table(r, seed, kf, kl)
                assert got[0].tolist() == want[0] and got[1].tolist() == want[1], (t, r, kf, kl)
