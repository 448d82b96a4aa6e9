"""bench.py's visible-token accounting (the basis of its FLOP and byte counts)
checked against the oracle's page manager, on the CPU."""
import bench
from oracle import OracleCache, OracleConfig, is_keyframe


def _host_cache(c, max_units):
    return OracleCache(OracleConfig(num_heads=1, head_dim=64, page_size=c["page"], patch_tokens=c["patch"],
                                    special_tokens=c["special"], num_scale_units=c["scale"],
                                    window_units=c["window"], max_units=max_units), with_pool=False)


def _visible(oc):
    return sum(oc.visible_table()[1])


def test_stream_visible_tokens_match_oracle():
    """LingBot-shaped stream: after frame t the table holds stream_lk(t) tokens."""
    c = bench.STREAM
    oc = _host_cache(c, c["frames"])
    for t in range(c["frames"]):
        oc.append()
        assert _visible(oc) == bench.stream_lk(t), t


def test_keyframe_rule_and_visible_tokens_match_oracle():
    """Keyframe stream: bench keeps the oracle's keyframes, and a frame attends to
    keyframe_lk(units kept before it + 1) tokens; rollbacks restore the count."""
    c = bench.KEYFRAME
    oc = _host_cache(c, 800)
    kept = 0
    for t in range(800):
        assert bench.keyframe_kept(t) == is_keyframe(t, c["scale"], c["interval"]), t
        oc.append()
        assert _visible(oc) == bench.keyframe_lk(kept + 1), t
        if bench.keyframe_kept(t):
            kept += 1
        else:
            oc.rollback()
        assert _visible(oc) == (bench.keyframe_lk(kept) if kept else 0), t
