"""Host logic of bench.py that needs no GPU: the warm-up rule, the refusal
of more than one GPU and the check of --rows."""
import argparse
import types

import bench


class _FakeCuda:
    def __init__(self):
        self.syncs = 0

    def synchronize(self):
        self.syncs += 1


def _torch():
    return types.SimpleNamespace(cuda=_FakeCuda())


def test_explicit_warmup_runs_exactly_that_many_steps():
    calls = []
    t = _torch()
    n = bench.warm_up(lambda: calls.append(1), argparse.Namespace(warmup=5), t)
    assert n == 5 and len(calls) == 5
    assert t.cuda.syncs >= 1  # the timed region starts on an idle stream
    calls.clear()
    assert bench.warm_up(lambda: calls.append(1), argparse.Namespace(warmup=0), t) == 0 and not calls


def test_default_warmup_covers_the_minimum_steps_and_time(monkeypatch):
    # a fake clock that advances 30 ms per step: the 200 ms floor needs 7 steps
    now = [0.0]
    monkeypatch.setattr(bench.time, "perf_counter", lambda: now[0])
    calls = []

    def step():
        calls.append(1)
        now[0] += 0.030

    t = _torch()
    n = bench.warm_up(step, argparse.Namespace(warmup=None), t)
    assert n == len(calls) == 7
    assert t.cuda.syncs == n  # each step is synchronised, so the wall time is the GPU's


def test_default_warmup_runs_at_least_three_long_steps(monkeypatch):
    now = [0.0]
    monkeypatch.setattr(bench.time, "perf_counter", lambda: now[0])

    def step():
        now[0] += 1.0  # one second per step: the step floor decides

    assert bench.warm_up(step, argparse.Namespace(warmup=None), _torch()) == bench.WARMUP_MIN_STEPS == 3


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


def test_rows_below_the_component_count_are_refused(capsys):
    # the recipes draw their initial means from K distinct rows
    assert bench.main(["--rows", "5", "--workload", "ref"]) == 2
    assert "--rows" in capsys.readouterr().err
