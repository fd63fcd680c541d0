"""bench.py's host-side contract (no GPU): one GPU only, the profiled
configuration is the default one, and the profile-derived HBM traffic is
reported only for that configuration."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _args(*argv):
    old = sys.argv
    sys.argv = ["bench.py", *argv]
    try:
        return bench.parse()
    finally:
        sys.argv = old


@pytest.mark.parametrize("n", ["2", "8"])
def test_more_than_one_gpu_exits_with_a_message(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", n], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_profiled_configuration_is_the_default():
    args = _args()
    for k, v in bench.PROFILED.items():
        assert getattr(args, k) == v, k


def test_traffic_only_for_the_profiled_configuration():
    t = bench.profiled_traffic(_args())
    assert t is None or (isinstance(t, int) and t > 0)  # None once the kernel sources change
    for argv in (["--tile", "256x128"], ["--split", "2"], ["--backend", "cu16"], ["--kslices", "4"], ["--lead", "0"],
                 ["--c-dtype", "bf16"], ["--layout", "kn"], ["--teams", "1"], ["--copy-store", "stream"]):
        assert bench.profiled_traffic(_args(*argv)) is None, argv


def test_single_row_option_names_every_row_function():
    """--row picks one of the other rows (a profiling aid); the default runs the bench line."""
    assert _args().row is None
    for r in ("rs", "ag70", "a2a", "attention"):
        assert _args("--row", r).row == r
    for fn in (bench.rs_rows, bench.ag70_row, bench.a2a_row, bench.attention_rows):
        assert callable(fn)
    with pytest.raises(SystemExit):
        _args("--row", "headline")


def test_interleaved_rows_pool_two_rounds_in_reverse_order(monkeypatch):
    """The other rows time their calls in two rounds, the second in reverse
    order, and report the median of both rounds' samples, so that a drift of
    the clock over the row weighs on every call alike."""
    seen = []

    class FakeTimer:
        def series(self, fn, steps, warmup, cold):
            name = fn()
            seen.append((name, warmup))
            base = {"a": 1.0, "b": 2.0, "c": 3.0}[name]
            drift = 0.1 * len(seen)  # later launches run slower
            return {"samples": [base + drift] * steps}

    monkeypatch.setattr(bench, "check", lambda ws, stream: None)
    calls = {k: ((lambda k=k: k), None) for k in ("a", "b", "c")}
    t = bench._interleaved_medians(FakeTimer(), None, calls, steps=3, warmup=2)
    assert [n for n, _ in seen] == ["a", "b", "c", "c", "b", "a"]
    assert [w for _, w in seen] == [2, 2, 2, 1, 1, 1]
    # each call's samples come from one early and one late slot: the drift is the same for all
    assert t["a"] - 1.0 == pytest.approx(t["b"] - 2.0) == pytest.approx(t["c"] - 3.0)
