"""bench.py's command-line contract on a machine without a GPU.

More than one GPU is refused with a message (the library has no multi-GPU path), and without a
device the benchmark exits with an error instead of printing a result line: nothing in it falls
back to the CPU.
"""
import json
import os
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def _run(*args):
    return subprocess.run([sys.executable, BENCH, *args], capture_output=True, text=True, timeout=300, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    out = _run("--gpus", "2")
    assert out.returncode == 2
    assert "one GPU" in out.stderr and out.stdout == ""


def test_no_result_line_without_a_gpu():
    if torch.cuda.device_count() > 0:  # counting devices does not initialise one
        pytest.skip("checks the behaviour without a GPU")
    out = _run("--no-secondary", "--steps", "2", "--warmup", "1", "--cpu-seconds", "0.1")
    assert out.returncode != 0
    assert "needs a GPU" in out.stderr
    assert out.stdout.strip() == "", "no JSON line may be printed without a device"


# ---------------------------------------------------------------------------
# The timing harness with a stub step and stub events: every run length the driver or a user
# may ask for (one step included) times without raising and samples the launches it says.
# ---------------------------------------------------------------------------
sys.path.insert(0, ROOT)
import bench  # noqa: E402


class _Handle:
    launch = None  # the timed launch that recorded this event


class _StubEvents:
    """Event handles with made-up times: timed launch j starts at j * 30 us and stops 28 us later."""

    made = []

    def __init__(self, n):
        self.ev = [_Handle() for _ in range(n)]
        self.closed = False
        _StubEvents.made.append(self)

    def elapsed_s(self, a, b):
        t = lambda i: self.ev[i].launch * 30e-6 + (28e-6 if i % 2 else 0.0)
        return t(b) - t(a)

    def close(self):
        self.closed = True


@pytest.mark.parametrize("steps", [1, 2, 5, 20, 33, 1024])
def test_timed_run_any_step_count(steps):
    calls = []

    def step(i, e0, e1):
        j = len(calls) - 5  # the timed launch's index (negative during the warmup)
        if e0 is not None:
            e0.launch = e1.launch = j
        calls.append((i, e0, e1))

    _StubEvents.made.clear()
    t = bench.Timed(lambda: None, events=_StubEvents).run(step, n_sets=6, warmup=5, steps=steps)
    every, sampled = bench.sampling_plan(steps)
    assert len(calls) == 5 + steps
    assert all(e0 is None for _, e0, _ in calls[:5]), "warmup steps record no events"
    timed = calls[5:]
    assert [n for n, (_, e0, _) in enumerate(timed) if e0 is not None] == sampled
    assert sampled[0] == 0 and sampled[-1] == steps - 1, "both ends of the timed region are sampled"
    assert [i for i, _, _ in calls] == [i % 6 for i in range(5 + steps)], "sets rotate in order"
    assert t["dispatch_events"] == len(sampled)
    assert t["intervals"] == len(sampled) - 1
    assert t["sample_every"] == every
    assert t["kernel_s"] > 0 and t["wall_s"] >= 0
    assert abs(t["dispatch_event_mean_s"] - 28e-6) < 1e-12
    # first start to last stop: (steps - 1) * 30 + 28 us over the steps
    assert abs(t["span_s"] - ((steps - 1) * 30e-6 + 28e-6) / steps) < 1e-12
    if steps == 1:
        assert t["interval_mean_s"] is None and t["kernel_s"] == t["dispatch_event_mean_s"]
    else:
        assert abs(t["interval_mean_s"] - 30e-6) < 1e-12
        assert t["kernel_s"] == min(t["dispatch_event_mean_s"], t["span_s"])
    assert _StubEvents.made and all(e.closed for e in _StubEvents.made)
    # the JSON fields of a run: microseconds, None where there is no interval
    f = bench.spread_fields(t)
    assert set(f) == {f"{k}_{q}_us" for k in ("dispatch_event", "interval") for q in ("median", "p10", "p90")}
    json.dumps(f)


def test_sampling_plan():
    assert bench.sampling_plan(1) == (1, [0])
    assert bench.sampling_plan(2) == (1, [0, 1])
    assert bench.sampling_plan(20) == (19, [0, 19])
    assert bench.sampling_plan(33) == (32, [0, 32])
    assert bench.sampling_plan(1024) == (32, list(range(0, 1024, 32)) + [1023])
    for steps in range(1, 300):
        every, sampled = bench.sampling_plan(steps)
        assert 1 <= every <= 32 and sampled[0] == 0 and sampled[-1] == steps - 1
        assert sampled == sorted(set(sampled))
        assert len(sampled) <= steps // every + 2
        assert steps > 33 or len(sampled) == min(steps, 2)
    with pytest.raises(ValueError):
        bench.sampling_plan(0)


def test_driver_arguments_parse():
    a = bench.parse_args(["--gpus", "1", "--steps", "20", "--warmup", "5"])
    assert (a.gpus, a.steps, a.warmup, a.no_secondary) == (1, 20, 5, False)
    with pytest.raises(SystemExit):
        bench.parse_args(["--steps", "0"])


def test_a_failing_secondary_leg_is_recorded():
    sec = {}
    bench.leg(sec, "ok", lambda: {"v": 1})
    bench.leg(sec, "bad", lambda: 1 / 0)
    assert sec["ok"] == {"v": 1}
    assert sec["bad"]["error"].startswith("ZeroDivisionError")


def test_host_cpu_info_states_the_cores():
    info = bench.host_cpu_info()
    assert info["host_cores"] == os.cpu_count()
    assert 1 <= info["share"] <= info["affinity_cores"]
    json.dumps(info)


def test_driver_command_reaches_the_device_check():
    """The driver's exact command parses and gets as far as asking for a device."""
    if torch.cuda.device_count() > 0:
        pytest.skip("checks the behaviour without a GPU")
    out = _run("--gpus", "1", "--steps", "20", "--warmup", "5")
    assert out.returncode != 0 and "needs a GPU" in out.stderr
    assert out.stdout.strip() == ""
