"""Host-side logic of bench.py that needs no GPU: the one-GPU refusal, the byte count behind the
selected-KV bandwidth, and the guard that drops the recorded HBM traffic once the scoring
kernel's sources change."""
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""          # no JSON line for a refused run


def test_selected_kv_bytes_counts_valid_tokens_of_kept_blocks():
    # two sequences of 130 and 64 tokens: blocks of 64, 64, 2 and 64 valid tokens
    idx = torch.tensor([[[0, 2, -1], [1, 2, 5]], [[0, -1, -1], [3, 0, -1]]], dtype=torch.int32)
    lens = np.array([130, 64])
    per_token = 128 * 2 * 2          # K and V, 128 dims, bf16
    want = (64 + 2) + (64 + 2) + 64 + 64   # entry 5 and block 3 of a one-block sequence are not attended
    assert bench.selected_kv_bytes(idx, lens) == want * per_token
    assert bench.selected_kv_bytes(idx, lens, elem=4) == 2 * want * per_token


def test_recorded_traffic_follows_the_kernel_sources(tmp_path, monkeypatch):
    rec = bench.recorded_traffic(67706880)
    if rec is None:
        pytest.skip("no traffic record for the current sources")
    assert 0.9 < rec["vs_algorithmic"] < 1.5
    assert rec["bytes_per_launch"] == rec["fetch_bytes"] + rec["write_bytes"]
    # a change to the kernel's sources voids the record
    changed = tmp_path / "score.hip"
    changed.write_text(open(os.path.join(ROOT, bench.SCORE_SOURCES[0])).read() + "\n// edited\n")
    monkeypatch.setattr(bench, "SCORE_SOURCES", (str(changed),) + tuple(bench.SCORE_SOURCES[1:]))
    assert bench.recorded_traffic(67706880) is None


def test_sources_digest_is_stable_and_content_based(tmp_path):
    a, b = tmp_path / "a.txt", tmp_path / "b.txt"
    a.write_text("x")
    b.write_text("x")
    assert bench.sources_digest([str(a)]) == bench.sources_digest([str(b)])
    b.write_text("y")
    assert bench.sources_digest([str(a)]) != bench.sources_digest([str(b)])


class _FakeCuda:
    """The parts of torch.cuda that bench.time_exact_steps touches, recording what runs when."""
    def __init__(self, log):
        self.log = log

    def synchronize(self):
        self.log.append("sync")

    class Event:
        def __init__(self, enable_timing=False):
            self.t = 0.0

        def record(self):
            pass

        def elapsed_time(self, other):
            return 1.0


@pytest.mark.parametrize("steps,warmup", [(20, 5), (400, 40), (450, 0), (1, 1), (199, 3), (201, 7)])
def test_exact_steps_and_warmup(monkeypatch, steps, warmup):
    """bench.time_exact_steps runs exactly `warmup` untimed calls, then replays graphs holding
    exactly `steps` calls in total (a full graph of up to 200, and a graph of the remainder)."""
    log = []
    calls = []

    class FakeTorch:
        cuda = _FakeCuda(log)

    class FakeGraph:
        def __init__(self, fn, n):
            self.fn, self.n = fn, n

        def replay(self):
            log.append("replay%d" % self.n)
            for i in range(self.n):
                calls.append(("timed", i))

    monkeypatch.setattr(bench, "timed_graph", lambda fn, n, torch, eager_first=True: FakeGraph(fn, n))

    def fn(i):
        calls.append(("eager", i))
    t = bench.time_exact_steps(fn, steps, warmup, FakeTorch)
    eager = [c for c in calls if c[0] == "eager"]
    timed = [c for c in calls if c[0] == "timed"]
    assert eager == [("eager", i) for i in range(warmup)]
    assert len(timed) == steps
    assert max(int(e[len("replay"):]) for e in log if e.startswith("replay")) <= bench.GRAPH_MAX_STEPS
    assert t == pytest.approx(1e-3 / steps)


def _undefined_globals(path):
    """(function, name) for every name a function reads as a global that the module never binds
    and that is not a builtin: the mistakes only a run of that function would otherwise show"""
    import builtins
    import symtable
    top = symtable.symtable(open(path).read(), path, "exec")
    bound = {s.get_name() for s in top.get_symbols() if s.is_assigned() or s.is_imported() or s.is_namespace()}
    bad = []

    def walk(t):
        for ch in t.get_children():
            for s in ch.get_symbols():
                name = s.get_name()
                if s.is_referenced() and s.is_global() and name not in bound and not hasattr(builtins, name):
                    bad.append((ch.get_name(), name))
            walk(ch)
    walk(top)
    return bad


@pytest.mark.parametrize("rel", ["bench.py", "__graft_entry__.py", "long_context_sparse_select_amd/__init__.py",
                                 "long_context_sparse_select_amd/_lib.py"])
def test_no_undefined_globals(rel):
    """bench.py's GPU paths (and the build / binding modules) never run on the CPU: a name read
    before it is bound anywhere would only surface as a NameError on the GPU"""
    path = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), rel)
    assert _undefined_globals(path) == []
