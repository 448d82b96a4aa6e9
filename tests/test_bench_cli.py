"""bench.py's argument handling and oracle legs, run on the CPU with the driver's arguments.

The harness runs `bench.py --gpus 1 --steps 20 --warmup 5`; these
tests run the same argument parsing and the same oracle (cpu_baseline) code
paths that command takes, at the sizes it takes them, without a GPU.
"""
import bench


def test_driver_arguments_give_the_full_size_chunked_line():
    a = bench.parse_args(["--gpus", "1", "--steps", "20", "--warmup", "5"])
    assert a.workload == "chunked" and a.steps == 20 and a.warmup == 5
    # --steps counts chunk steps; the shapes stay those of the chunked workload
    assert bench.chunk_tokens() == 10992
    assert bench.CHUNK["window_chunks"] * bench.chunk_tokens() == 43968
    assert bench.CHUNK["layers"] == 24 and bench.CHUNK["heads"] == 16
    # the warm-up fills the window before any timed step
    assert max(a.warmup, bench.CHUNK["window_chunks"]) >= bench.CHUNK["window_chunks"]
    d = bench.parse_args([])
    assert d.workload == "chunked" and d.steps == 20


def test_stream_steps_time_the_tail_of_the_full_stream():
    a = bench.parse_args(["--workload", "stream", "--steps", "20", "--warmup", "5"])
    assert a.steps == 20
    # the stream stays 1,000 frames; the last 20 are timed
    assert bench.STREAM["frames"] == 1000
    assert bench.stream_lk(bench.STREAM["frames"] - 1) == 24432


def test_chunked_oracle_leg_runs():
    """The chunked cpu_baseline leg (smaller query slice): the window holds 43,968 keys."""
    sec, flops, lk = bench.oracle_chunked_sample(query_rows=8)
    assert lk == 43968
    assert flops == bench.attn_flops(8, 43968, 16)
    assert sec > 0


def test_stream_oracle_leg_with_driver_arguments():
    """The stream extra's cpu_baseline leg at its default sample (a regression test for a sample larger
    than the frames streamed).  Sizes the oracle cache for every frame it appends."""
    a = bench.parse_args(["--gpus", "1", "--steps", "20", "--warmup", "5"])
    sec, flops, n = bench.oracle_stream_sample(bench.STREAM["frames"], a.cpu_sample)
    assert n == a.cpu_sample and sec > 0
    assert flops == sum(bench.attn_flops(262, bench.stream_lk(t), 16) for t in range(1000 - n, 1000))
    # a sample larger than the stream is clamped, not an error
    sec, flops, n = bench.oracle_stream_sample(6, 40)
    assert n == 6


def test_host_info_names_cores_and_blas():
    h = bench.host_info()
    assert h["cores"] >= 1 and h["blas_threads"] >= 1
    assert h["cpu_model"] and h["blas"]


def test_windowed_arguments_and_oracle_leg():
    """--workload windowed: 25,000 frames by default (the pages' long indoor run); the oracle leg times
    frames around the first restart, which falls where the 129th kept unit is appended."""
    a = bench.parse_args(["--workload", "windowed"])
    assert a.steps == 25000 and a.replay_frames == 2000
    c = bench.WINDOWED
    sched = bench.windowed_schedule(600)
    first = next(t for t, (_, r) in enumerate(sched) if r)
    assert sum(bench.keyframe_kept(t, c) for t in range(first)) == c["slots"]
    sec, flops, t0 = bench.oracle_windowed_sample(4)
    assert t0 == first - 2 and sec > 0
    assert flops == sum(bench.attn_flops(262, bench.keyframe_lk(sched[t][0], c), 16) for t in range(t0, t0 + 4))
