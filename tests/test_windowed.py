"""Windowed inference (restart per window, shared overlap units): library tables bit-exact against the oracle."""
import pytest

from oracle import OracleCache, OracleConfig, OracleWindowed, is_keyframe, required_pages
from paged_sliding_window_kv_amd import KvCache, WindowedStream


@pytest.mark.parametrize("window_slots,overlap,interval", [(128, 16, 2), (40, 0, 1), (7, 6, 3)])
def test_windowed_25000_frames_host_tables(window_slots, overlap, interval):
    """25,000 frames (the page's long indoor run) through the LingBot cache shape, host metadata only."""
    S, W, P, X = 8, 64, 256, 6
    ocfg = OracleConfig(num_heads=1, head_dim=64, patch_tokens=P, special_tokens=X, num_scale_units=S,
                        window_units=W, max_units=window_slots + 1)
    oc = OracleWindowed(OracleCache(ocfg, with_pool=False), window_slots, overlap)
    hc = KvCache(num_heads=1, patch_tokens=P, special_tokens=X, num_scale_units=S, window_units=W,
                 max_units=window_slots + 1)
    ws = WindowedStream(hc, window_slots, overlap)
    assert hc.num_pages == required_pages(ocfg)
    max_special = 0
    for t in range(25000):
        r1 = oc.append()
        r2 = ws.append()
        assert r1 == r2
        if is_keyframe(t, S, interval):
            oc.keep()
            ws.keep()
        else:
            if t % 997 == 0:
                assert hc.visible_table()[0].tolist() == oc.cache.visible_table()[0]
            oc.drop()
            ws.drop()
        st = hc.state()
        max_special = max(max_special, len(st["special_pages"]))
        if t % 1999 == 0:
            ids, lens = hc.visible_table()
            oids, olens = oc.cache.visible_table()
            assert ids.tolist() == oids and lens.tolist() == olens
            assert st == oc.cache.state()
    assert ws.windows == oc.windows > 0
    # memory bound: the special stream restarts with every window
    assert max_special <= -(-(window_slots + 1) // (P // X))
