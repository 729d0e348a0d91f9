"""bench.py's command line on the CPU: more than one GPU is refused with a
message (one process per GPU is not this bench's shape: the step shards by
sequence with no exchange), before anything touches a GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2", "--steps", "1"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and r.stdout == ""


def test_torch_events_need_one_stream():
    """torch's events time torch's current stream only, so they are refused
    with the default two batches in flight (each on its own stream)."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--torch-events", "--steps", "1"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "--streams 1" in r.stderr and r.stdout == ""


def test_copies_are_a_multiple_of_the_streams():
    """Copy j is always stepped on stream j % streams, so the state copies
    come in whole multiples of the streams."""
    sys.path.insert(0, ROOT)
    import argparse
    import bench
    for streams in (1, 2, 3, 4):
        for copies in (0, 1, 2, 5):
            a = argparse.Namespace(copies=copies, streams=streams)
            R = bench.n_copies(a, [1 << 28, 1 << 28, 0])
            assert R % streams == 0 and R >= copies and (copies or R >= 2)
