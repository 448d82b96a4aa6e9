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


def test_chunked_and_global_visible_tokens_match_oracle():
    """Chunked: after the window fills, a chunk attends to window_chunks x chunk tokens.
    Global (no window): after 100 frames all 137,400 tokens are visible."""
    tokens = bench.CHUNK["frames_per_chunk"] * bench.VGGT_TOKENS
    W = bench.CHUNK["window_chunks"]
    oc = OracleCache(OracleConfig(num_heads=1, head_dim=64, page_size=bench.CHUNK["page"], patch_tokens=tokens,
                                  special_tokens=0, num_scale_units=0, window_units=W, max_units=W + 3),
                     with_pool=False)
    for i in range(W + 3):
        oc.append()
        assert _visible(oc) == min(i + 1, W) * tokens
    og = OracleCache(OracleConfig(num_heads=1, head_dim=64, page_size=256, patch_tokens=bench.VGGT_TOKENS,
                                  special_tokens=0, num_scale_units=0, window_units=0, max_units=100),
                     with_pool=False)
    for _ in range(100):
        og.append()
    assert _visible(og) == 100 * bench.VGGT_TOKENS == 137400


def test_profile_hash_ignores_comments_only():
    """The hash that ties committed counter summaries to the kernel source sees code, not comments."""
    src = 'int a = 1;  // one\n// a comment line\n\nconst char* s = "x // y";  /* kept */\n'
    assert bench.code_text(src, "//") == 'int a = 1;\nconst char* s = "x // y";  /* kept */'
    assert bench.code_text("x = 1  # note\n# only\ny = '#'\n", "#") == "x = 1\ny = '#'"
    assert bench.code_text("a = 1\n", "//") != bench.code_text("a = 2\n", "//")


def test_windowed_schedule_matches_the_c_driver():
    """Windowed stream: bench's per-frame unit count and restart flag follow libkvc's windowed driver on a
    host-only cache of the benched shape, and a frame attends to keyframe_lk(units) tokens."""
    from paged_sliding_window_kv_amd import KvCache, WindowedStream
    c = bench.WINDOWED
    frames = 1200
    hc = KvCache(num_heads=1, patch_tokens=c["patch"], special_tokens=c["special"], num_scale_units=c["scale"],
                 window_units=c["window"], max_units=c["slots"] + 1)
    ws = WindowedStream(hc, c["slots"], c["overlap"])
    sched = bench.windowed_schedule(frames)
    for t, (units, restart) in enumerate(sched):
        assert ws.append() == restart, t
        assert hc.state()["num_units"] == units, t
        assert int(hc.visible_table()[1].sum()) == bench.keyframe_lk(units, c), t
        if bench.keyframe_kept(t, c):
            ws.keep()
        else:
            ws.drop()
    assert ws.windows == sum(r for _, r in sched) >= 4
