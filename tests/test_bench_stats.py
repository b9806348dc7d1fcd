"""The benchmark's arithmetic, with no GPU: best-of / median / mean selection
and the run loop driven by a scripted fake clock ("Day 20: the number the
Triton kernel has to beat", sections "What I added today" and "What I
learned": best-of is the headline, mean and median show the spread), the
event-interval and rate conversions, and the CPU baseline record."""

import os

import pytest

import bench


class FakeClock:
    """Returns scripted instants; each call to fn advances it by the next
    scripted duration."""

    def __init__(self, durations):
        self.t = 100.0
        self.durations = list(durations)
        self.calls = 0

    def __call__(self):
        return self.t

    def work(self):
        self.t += self.durations[self.calls % len(self.durations)]
        self.calls += 1


def test_time_runs_stops_after_the_budget():
    clk = FakeClock([0.25, 0.125, 0.375])
    times = bench.time_runs(clk.work, 1.0, clock=clk)
    # 0.25 + 0.125 + 0.375 = 0.75 < 1.0; the fourth call reaches the budget.
    assert times == [0.25, 0.125, 0.375, 0.25]


def test_time_runs_takes_the_minimum_number_of_runs():
    clk = FakeClock([5.0])
    times = bench.time_runs(clk.work, 1.0, clock=clk, min_runs=3)
    assert times == pytest.approx([5.0, 5.0, 5.0])


def test_run_stats_best_median_mean():
    st = bench.run_stats([0.004, 0.001, 0.003, 0.010, 0.002])
    assert st == pytest.approx({"best": 0.001, "median": 0.003, "mean": 0.004, "runs": 5})
    even = bench.run_stats([4.0, 1.0, 3.0, 2.0])
    assert even["median"] == pytest.approx(2.5) and even["best"] == 1.0


def test_best_of_is_not_the_mean():
    """A slow outlier (a preempted run) moves the mean, not the best-of."""
    st = bench.run_stats([1.0] * 9 + [100.0])
    assert st["best"] == 1.0 and st["median"] == 1.0 and st["mean"] == pytest.approx(10.9)


def test_per_step_and_rate():
    assert bench.per_step_us(12.5, 100) == pytest.approx(125.0)
    # The headline's 8 MiB of K/V in 8 µs.
    assert bench.rate(8 << 20, 8.0) == pytest.approx(1048.576)
    assert bench.rate(38_663_094_272, 61.747, 1e12) == pytest.approx(626.15, rel=1e-4)


def test_cpu_record_states_the_cores():
    rec = bench.cpu_record(1.5, "GB/s", "sample", 4, extra=1)
    assert rec["cores"] == 4 and rec["kind"] == "oracle" and rec["extra"] == 1
    assert rec["cores_available"] == len(os.sched_getaffinity(0))
    assert rec["cpu_count"] == os.cpu_count()
