"""Host logic of bench.py's timers, with stand-in events (no GPU): a launch in
its own event pair counts the pair's time; launches issued back to back in one
pair count a share each; events return to the pool after collection; and
`--gpus N` with N > 1 exits with a message."""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))
import bench  # noqa: E402


class FakeEvent:
    """Records a 'timestamp' from a shared clock the test advances."""

    def __init__(self, clock):
        self.clock = clock
        self.t = None

    def record(self):
        self.t = self.clock[0]

    def elapsed_time(self, other):  # milliseconds, as torch's events report
        return other.t - self.t


def fake_timer():
    clock = [0.0]
    timer = bench.KernelTimer()
    timer._event = lambda: FakeEvent(clock)
    return timer, clock


def test_run_counts_each_pair():
    timer, clock = fake_timer()

    def launch(ms):
        def fn():
            clock[0] += ms
            return ms
        return fn
    assert timer.run("a", launch(2.0)) == 2.0
    timer.run("a", launch(4.0))
    timer.run("b", launch(1.0))
    timer.collect()
    assert timer.times["a"] == [pytest.approx(2e-3), pytest.approx(4e-3)]
    assert timer.times["b"] == [pytest.approx(1e-3)]
    assert timer.mean("a") == pytest.approx(3e-3)
    assert len(timer.pool) == 6 and timer.pending == []


def test_run_many_shares_one_pair():
    timer, clock = fake_timer()

    def step(k):
        def fn():
            clock[0] += 0.5 * (k + 1)
            return k
        return fn
    outs = timer.run_many("m", [step(k) for k in range(4)])
    assert outs == [0, 1, 2, 3]
    timer.collect()
    # one pair around 0.5 + 1.0 + 1.5 + 2.0 ms: four calls of 1.25 ms each
    assert timer.times["m"] == [pytest.approx(1.25e-3)] * 4
    assert timer.median("m") == pytest.approx(1.25e-3)


def test_pool_is_used_before_new_events():
    timer, clock = fake_timer()
    timer._event = bench.KernelTimer._event.__get__(timer)  # the real pool logic
    pooled = [FakeEvent(clock) for _ in range(4)]
    timer.pool = list(pooled)
    timer.run("x", lambda: None)
    timer.run("x", lambda: None)
    assert timer.pool == [] and all(e.t is not None for e in pooled)


def test_no_timer_and_capture_timer_run_many():
    assert bench._NoTimer().run_many("k", [lambda: 1, lambda: 2]) == [1, 2]
    cap = bench._CaptureTimer()
    fns = [lambda: 3, lambda: 4]
    assert cap.run_many("k", fns) == [3, 4]
    assert cap.fns["k"] is fns[-1]


def test_more_than_one_gpu_exits():
    r = subprocess.run([sys.executable, os.path.join(os.path.dirname(HERE), "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
